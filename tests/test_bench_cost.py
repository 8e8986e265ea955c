"""The bench's cost model and command line, on the CPU.

The algorithmic byte counts are the ring's own: a reduce-scatter round reads
two chunks and writes one, an all-gather round reads one and writes one
("全归约 3：Ring——每步大小恒定", cost card: 2 (P - 1) / P N per rank over
2 (P - 1) rounds), at the widths the kernels use (the bf16 all-reduce carries
its partial sums in fp32).  The MLP's flops are the TPU chapter's closed
form.
"""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_all_reduce_bytes():
    # P = 8, 64 Mi fp32 per rank: 7 rounds of 12 B and 7 of 8 B per chunk element
    P, n = 8, 64 << 20
    C = n // P
    assert bench.moved_bytes("all_reduce", P, n, "f32") == 7 * 8 * C * (12 + 8) == 9_395_240_960
    assert bench.moved_bytes("reduce_scatter", P, n, "f32") == 7 * 8 * C * 12
    assert bench.moved_bytes("all_gather", P, n, "f32") == 7 * 8 * C * 8


def test_bf16_all_reduce_bytes():
    # P = 16, 128 Mi bf16: round 0 reads 2 + 2 and writes 4; middle rounds read
    # 2 + 4 and write 4; the owner's round writes 2; the gather moves 2 + 2
    P, n = 16, 128 << 20
    C = n // P
    rs = C * P * ((2 + 2 + 4) + 13 * (2 + 4 + 4) + (2 + 4 + 2))
    ag = 15 * C * P * 4
    assert bench.moved_bytes("all_reduce", P, n, "bf16") == rs + ag == 27_648_851_968


def test_other_workloads_bytes():
    P, n = 8, 64 << 20
    C = n // P
    assert bench.moved_bytes("ppermute", 2, n, "f32") == 2 * 2 * n * 4
    assert bench.moved_bytes("psum_circulating", P, n, "f32") == 2 * (P + 1) * n * 4 * P == 38_654_705_664
    assert bench.moved_bytes("reduce_scatter_bidir", P, n, "f32") == 7 * 12 * C * P + 8 * C * P
    assert bench.moved_bytes("all_reduce", 1, n, "f32") == 0


def test_mlp_cost_scales_with_tokens():
    small = bench.mlp_layer_cost(P=4, M=256, D=1024, F=16384)
    big = bench.mlp_layer_cost(P=4, M=8192, D=1024, F=16384)
    assert big["flop"] == 32 * small["flop"] == 549_755_813_888


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "ONE GPU" in r.stderr and r.stdout == ""


def test_every_workload_names_a_profiled_kernel_source():
    for k, files in bench.KERNEL_SOURCE.items():
        for f in files:
            assert os.path.exists(os.path.join(ROOT, "ring_collectives_amd", "csrc", f)), (k, f)
    assert len(bench._sha_source("tp_mlp_layer")) == 64


def test_kernel_name_follows_the_low_latency_limit():
    """The bench names ring_ll_kernel exactly for the one-way collectives
    whose chunks take the low-latency rounds (at most 256 KiB, words within
    64 MiB, the tuning knob not lower), and the library's workspace size
    agrees on which shapes hold the words."""
    from ring_collectives_amd import _native as N
    old = N.get_tuning()
    try:
        assert bench._ring_kernel("all_reduce", 4, 4096, "f32") == "ring_ll_kernel"
        assert bench._ring_kernel("reduce_scatter", 8, 8192, "i32") == "ring_ll_kernel"
        assert bench._ring_kernel("all_gather", 4, 4 * (128 << 10), "bf16") == "ring_ll_kernel"
        assert bench._ring_kernel("all_reduce", 4, 4 * ((64 << 10) + 4), "f32") == "ring_step_kernel"
        assert bench._ring_kernel("all_reduce", 8, 64 << 20, "f32") == "ring_step_kernel"
        assert bench._ring_kernel("reduce_scatter_bidir", 4, 4096, "f32") == "ring_bidir_kernel"
        assert bench._ring_kernel("ppermute", 2, 4096, "f32") == "copy_kernel_tab"
        N.set_tuning(ll_max_chunk_bytes=0)
        assert bench._ring_kernel("all_reduce", 4, 4096, "f32") == "ring_step_kernel"
    finally:
        N.set_tuning(**old)
    L = N.lib()
    with_words = L.ring_workspace_bytes(N.OP_ALL_REDUCE, 4, 4 * (64 << 10), N.RING_F32)
    without = L.ring_workspace_bytes(N.OP_ALL_REDUCE, 4, 4 * ((64 << 10) + 4), N.RING_F32)
    assert with_words > without


@pytest.mark.parametrize("P,n", [(8, 8 * 4096 * 3), (16, 16 * 2048), (3, 3 * 1000)])
def test_multi_thread_oracle_leg_keeps_the_bits(P, n):
    """The bench's multi-thread oracle leg runs the unchanged oracle on
    sub-problems made of one slice of every chunk: chunk c of a sub-problem
    holds only elements of chunk c, so the ring's order, and every bit, is
    the single call's (fp32, bf16, int32; all-reduce and reduce-scatter)."""
    import numpy as np
    import oracle
    from ring_collectives_amd import inputs
    T = bench._slice_threads(n // P, 8)
    assert (n // P) % T == 0 and T >= 1
    x = inputs.normal_f32(P, n, seed=2)
    xb = inputs.normal_bf16(P, n, seed=3)
    xi = np.random.default_rng(1).integers(-1000, 1000, size=(P, n), dtype=np.int32)
    for fn, a in ((oracle.all_reduce, x), (oracle.reduce_scatter, x), (oracle.all_reduce_bf16, xb),
                  (oracle.all_reduce, xi)):
        np.testing.assert_array_equal(bench._oracle_sliced(fn, a, P, T).view(np.uint8), fn(a).view(np.uint8))

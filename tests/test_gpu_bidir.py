"""GPU parity of the bidirectional ring reduce-scatter against the CPU oracle
("Pallas TPU Distributed Collectives 复习文档", section 4), through the C ABI.

fp32 and int32: every element of every rank buffer bit for bit -- the owner
chunks and every partial sum the schedule leaves behind (each half of every
other chunk is written exactly once).  bf16: the owner chunks bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_collectives_amd import _native as N
from ring_collectives_amd import collectives as rc
from ring_collectives_amd import inputs

from _gpu_helpers import bits, empty_ranks, note, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()
    yield


@pytest.fixture(autouse=True)
def _default_tuning():
    old = N.get_tuning()
    yield
    N.set_tuning(**old)


def _run(x, kind, in_place=False, ws=None):
    src = to_dev(x, kind)
    dst = src if in_place else empty_ranks(x.shape[0], x.shape[1], kind)
    ws = rc.reduce_scatter_bidir(src, dst, ws=ws)
    got = to_host(dst, kind)
    assert rc.last_error(ws)[0] == 0
    return got


@pytest.mark.parametrize("P", [2, 3, 4, 8])
def test_bidir_int32(P):
    note("bidir int32 P=%d" % P)
    x = inputs.to_chunk_major(inputs.ring_i32(P), P)
    got = _run(x, "i32")
    np.testing.assert_array_equal(got, oracle.reduce_scatter_bidir(x))
    C = x.shape[1] // P
    total = x.astype(np.int64).sum(axis=0)
    for r in range(P):
        np.testing.assert_array_equal(got[r, r * C:(r + 1) * C], total[r * C:(r + 1) * C])


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("C", [1, 7, 2048 * 3 + 100, 2048 * 5, 2048 * 4 + 8])
def test_bidir_f32_sizes(P, C):
    """Chunks whose halves do or do not start on a 16-byte boundary (vector
    or scalar path), tiny chunks (an empty bottom half at C = 1)."""
    note("bidir f32 P=%d C=%d" % (P, C))
    x = inputs.normal_f32(P, P * C, seed=90 + C % 89)
    np.testing.assert_array_equal(bits(_run(x, "f32")), bits(oracle.reduce_scatter_bidir(x)))


@pytest.mark.parametrize("P", [4, 8])
def test_bidir_in_place(P):
    note("bidir in place P=%d" % P)
    x = inputs.normal_f32(P, P * 40000, seed=91)
    np.testing.assert_array_equal(bits(_run(x, "f32", in_place=True)),
                                  bits(oracle.reduce_scatter_bidir(x)))


def test_bidir_page_trace_order():
    """The P = 4 walk-through's owner-first order on wide-range data: every
    partial sum the oracle pins to the page's table, bit for bit."""
    P, C = 4, 4096
    rng = np.random.default_rng(92)
    x = (rng.standard_normal((P, P * C)) * np.exp2(rng.integers(-20, 20, size=(P, P * C)))).astype(np.float32)
    note("bidir page trace order")
    np.testing.assert_array_equal(bits(_run(x, "f32")), bits(oracle.reduce_scatter_bidir(x)))


@pytest.mark.parametrize("P", [2, 4, 16])
@pytest.mark.parametrize("C", [8, 4096 * 3, 2048 * 2 + 24])
def test_bidir_bf16(P, C):
    note("bidir bf16 P=%d C=%d" % (P, C))
    x = inputs.normal_bf16(P, P * C, seed=93 + P)
    got = _run(x, "bf16")
    want, _ = oracle.reduce_scatter_bidir_bf16(x)
    for r in range(P):
        np.testing.assert_array_equal(got[r, r * C:(r + 1) * C], want[r, r * C:(r + 1) * C],
                                      err_msg="rank %d" % r)


def test_bidir_tuning_and_stepwise():
    """Tile size, wave mapping and the one-launch-per-step debug mode change
    nothing in the bits."""
    P = 8
    x = inputs.normal_f32(P, P * 70000, seed=94)
    want = oracle.reduce_scatter_bidir(x)
    for tv, mm in ((4, 0), (16, 2), (8, 2)):
        note("bidir tuning tile_vecs=%d map=%d" % (tv, mm))
        N.set_tuning(tile_vecs=tv, map_mode=mm)
        np.testing.assert_array_equal(bits(_run(x, "f32")), bits(want))
    note("bidir stepwise")
    N.set_tuning(tile_vecs=8, map_mode=0, stepwise=1)
    np.testing.assert_array_equal(bits(_run(x, "f32")), bits(want))


def test_bidir_repeated_calls_one_workspace():
    P = 4
    x = inputs.normal_f32(P, P * 20000, seed=95)
    ws = rc.workspace(N.OP_REDUCE_SCATTER_BIDIR, P, x.shape[1], torch.float32)
    want = oracle.reduce_scatter_bidir(x)
    for i in range(3):
        note("bidir repeated call %d" % i)
        np.testing.assert_array_equal(bits(_run(x, "f32", ws=ws)), bits(want))


def test_bidir_errors():
    P = 4
    x = to_dev(inputs.normal_f32(P, P * 4096, seed=96), "f32")
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(N.RingError) as e:
        rc.reduce_scatter_bidir(x, x, ws=small)
    assert e.value.code == N.RING_EWORKSPACE
    odd = [torch.zeros(4097, device="cuda") for _ in range(P)]
    with pytest.raises(N.RingError) as e:
        rc.reduce_scatter_bidir(odd, odd)
    assert e.value.code == N.RING_EINVAL


def test_bidir_watchdog_reports_timeout():
    """Rank 0 never signals step 2: the waits on it (rank 3 for top halves,
    rank 1 for bottom halves) and the ones behind them end in RING_ETIMEOUT."""
    P = 4
    x = inputs.normal_f32(P, P * 4096 * 4, seed=97)
    src = to_dev(x, "f32")
    dst = empty_ranks(P, x.shape[1], "f32")
    ws = rc.workspace(N.OP_REDUCE_SCATTER_BIDIR, P, x.shape[1], torch.float32)
    note("bidir watchdog drop_round=2")
    N.set_tuning(drop_round=2, timeout_s=0.05)
    rc.reduce_scatter_bidir(src, dst, ws=ws)
    code, info = rc.last_error(ws)
    assert code == N.RING_ETIMEOUT
    rank, rnd = info & 0xFF, (info >> 8) & 0xFF
    i = rnd - 2
    assert 0 <= i <= P - 3 and rank in ((0 - 1 - i) % P, (0 + 1 + i) % P), (rank, rnd)
    N.set_tuning(drop_round=0, timeout_s=5.0)
    rc.workspace_init(ws)
    rc.reduce_scatter_bidir(src, dst, ws=ws)
    assert rc.last_error(ws) == (0, 0)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.reduce_scatter_bidir(x)))


def test_bidir_full_size_fp32_p8_64Mi():
    """P = 8, 64 Mi fp32 per rank (the bandwidth workload's inputs) in the
    default launch configuration: every element bit for bit."""
    P, n = 8, 64 << 20
    note("bidir full size generate")
    x = inputs.normal_f32(P, n, seed=inputs.SEED_F32_BW)
    note("bidir full size run")
    got = _run(x, "f32")
    np.testing.assert_array_equal(bits(got), bits(oracle.reduce_scatter_bidir(x)))

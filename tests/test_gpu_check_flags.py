"""GPU tests of the check_flags debug knob ("全归约 3：Ring——每步大小恒定",
Walkthrough: every signal row is notified once per round and waited on with
Ge(1); here every flag of a launch is set exactly once and cleared by its
reader).  With the knob on, every flag set returns the flag's old value,
which must be 0, and every low-latency word must be empty before it is
written; a violation is reported as RING_EPROTOCOL.  The headline shapes and
every kernel kind run with the knob on and must stay error-free and equal to
the oracle bit for bit; a workspace whose flags were left set by a timed-out
call (and whose error word alone was cleared) must trip it."""
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
def _checked():
    old = N.set_tuning(check_flags=1)
    yield
    N.set_tuning(**old)


def test_headline_all_reduce_fp32():
    """P = 8, 64 Mi fp32 per rank, normal(0, 1), seed 2."""
    P, n = 8, 64 << 20
    note("check_flags: all-reduce fp32 P=8 64Mi")
    x = inputs.normal_f32(P, n, seed=2)
    dst = empty_ranks(P, n, "f32")
    ws = rc.all_reduce(to_dev(x, "f32"), dst)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))


def test_gradient_bucket_all_reduce_bf16():
    """P = 16, 128 Mi bf16 per rank, normal(0, 0.01), seed 3."""
    P, n = 16, 128 << 20
    note("check_flags: all-reduce bf16 P=16 128Mi")
    x = inputs.normal_bf16(P, n, seed=3)
    dst = empty_ranks(P, n, "bf16")
    ws = rc.all_reduce(to_dev(x, "bf16"), dst)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(to_host(dst, "bf16"), oracle.all_reduce_bf16(x))


@pytest.mark.parametrize("kind,op", [("f32", "all_reduce"), ("i32", "reduce_scatter"), ("i32", "all_gather"),
                                     ("bf16", "all_reduce")])
def test_small_calls_low_latency_rounds(kind, op):
    """The small configurations, in the low-latency rounds (each word must
    be empty when it is written)."""
    P = 4 if kind != "i32" else 8
    if kind == "i32":
        x = inputs.to_chunk_major(inputs.ring_i32(P), P)
    elif kind == "f32":
        x = inputs.to_chunk_major(inputs.small_f32(P, (8, 512)), P)
    else:
        x = inputs.normal_bf16(P, 4 * 4096, seed=31)
    n = x.shape[1]
    note("check_flags: %s %s P=%d n=%d" % (op, kind, P, n))
    src = to_dev(x, kind)
    dst = empty_ranks(P, n, kind)
    if op == "all_gather":
        C = n // P
        for r in range(P):
            dst[r][r * C:(r + 1) * C].copy_(src[r][r * C:(r + 1) * C])
        ws = rc.all_gather(dst)
        want = oracle.all_gather(x)
    elif op == "reduce_scatter":
        ws = rc.reduce_scatter(src, dst)
        want = oracle.reduce_scatter(x)
    else:
        ws = rc.all_reduce(src, dst)
        want = oracle.all_reduce_bf16(x) if kind == "bf16" else oracle.all_reduce(x)
    assert rc.last_error(ws)[0] == 0
    got = to_host(dst, kind)
    if op == "reduce_scatter":
        C = n // P
        for r in range(P):
            np.testing.assert_array_equal(got[r, r * C:(r + 1) * C], want[r, r * C:(r + 1) * C])
    else:
        np.testing.assert_array_equal(bits(got), bits(want))


def test_bidirectional_and_circulating_psum():
    P, n = 8, 8 << 20
    x = inputs.normal_f32(P, n, seed=33)
    src = to_dev(x, "f32")
    note("check_flags: bidirectional reduce-scatter P=8 8Mi")
    dst = empty_ranks(P, n, "f32")
    ws = rc.reduce_scatter_bidir(src, dst)
    assert rc.last_error(ws)[0] == 0
    got, want = to_host(dst, "f32"), oracle.reduce_scatter_bidir(x)
    C = n // P
    for r in range(P):
        np.testing.assert_array_equal(bits(got[r, r * C:(r + 1) * C]), bits(want[r, r * C:(r + 1) * C]))
    note("check_flags: circulating psum P=8 8Mi")
    dst = empty_ranks(P, n, "f32")
    ws = rc.psum_circulating(src, dst)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.psum_circulating(x)[0]))


def _bf16_dev(a):
    return [torch.from_numpy(np.ascontiguousarray(a[q]).view(np.int16)).cuda().view(torch.bfloat16)
            for q in range(a.shape[0])]


@pytest.mark.parametrize("bn", [256, 128])
def test_fused_gemms_full_occupancy(bn):
    """GEMM + reduce-scatter and all-gather + GEMM at M = N = 4096, P = 4,
    integer-valued operands (exact in any order), every element."""
    N.set_tuning(gemm_tile_n=bn)
    P, M, Nn, K = 4, 4096, 4096, 256
    rng = np.random.default_rng(930)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    note("check_flags: gemm_rs P=4 4096x4096x256 tile_n=%d" % bn)
    out = [torch.empty((M // P, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws = rc.gemm_reduce_scatter(_bf16_dev(A), _bf16_dev(B), out)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(np.stack([o.cpu().numpy() for o in out]).view(np.uint32),
                                  oracle.gemm_reduce_scatter(A, B).view(np.uint32))
    As = A[:, :M // P]
    note("check_flags: ag_gemm P=4 4096x4096x256 tile_n=%d" % bn)
    full = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    C = [torch.empty((M, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws = rc.all_gather_gemm(_bf16_dev(As), _bf16_dev(B), full, C)
    assert rc.last_error(ws)[0] == 0
    want_full, want_c = oracle.all_gather_gemm(As, B)
    np.testing.assert_array_equal(np.stack([c.cpu().numpy() for c in C]).view(np.uint32), want_c.view(np.uint32))


@pytest.mark.parametrize("M", [1024, 256])
def test_mlp_layer(M):
    """The MLP layer, fused (1024 tokens) and unfused (256), on operands
    whose every sum is exact (x rows of three ones, W1 in {0, 1}, W2 in
    {-1, 0, 1})."""
    P, D, F = 4, 256, 1024
    rng = np.random.default_rng(931)
    x = np.zeros((P, M // P, D), dtype=np.float32)
    for q in range(P):
        for i in range(M // P):
            x[q, i, rng.choice(D, size=3, replace=False)] = 1.0
    w1 = rng.integers(0, 1, size=(P, D, F // P), endpoint=True).astype(np.float32)
    w2 = rng.integers(-1, 1, size=(P, F // P, D), endpoint=True).astype(np.float32)
    x, w1, w2 = (inputs.bf16_bits(a) for a in (x, w1, w2))
    bf = torch.bfloat16
    full = [torch.empty((M, D), dtype=bf, device="cuda") for _ in range(P)]
    h = [torch.empty((M, F // P), dtype=bf, device="cuda") for _ in range(P)]
    out = [torch.empty((M // P, D), dtype=bf, device="cuda") for _ in range(P)]
    note("check_flags: tp_mlp P=4 M=%d" % M)
    ws = rc.tp_mlp_layer(_bf16_dev(x), _bf16_dev(w1), _bf16_dev(w2), full, h, out)
    assert rc.last_error(ws)[0] == 0
    _, _, want = oracle.tp_mlp_layer(x, w1, w2)
    got = np.stack([t.view(torch.int16).cpu().numpy().view(np.uint16) for t in out])
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("ll_max", [0, 262144])
def test_flags_left_set_trip_the_check(ll_max):
    """A call whose rank 0 never signals round 1 times out and leaves flags
    (or words) set; with only the error word cleared, the next call on that
    workspace finds a flag already set where it sets one and reports
    RING_EPROTOCOL.  Every wait still ends: a flag left set only lets a wait
    pass early.  After a full zero fill the call is clean again."""
    N.set_tuning(ll_max_chunk_bytes=ll_max)
    P, n = 4, 4 * 8192
    x = inputs.normal_f32(P, n, seed=932)
    src = to_dev(x, "f32")
    ws = rc.workspace(N.OP_ALL_REDUCE, P, n, torch.float32)
    note("check_flags: dropped signal, ll_max=%d" % ll_max)
    N.set_tuning(drop_round=1, timeout_s=0.05, check_flags=0)
    rc.all_reduce(src, empty_ranks(P, n, "f32"), ws=ws)
    assert rc.last_error(ws)[0] == N.RING_ETIMEOUT
    N.set_tuning(drop_round=0, timeout_s=5.0, check_flags=1)
    ws[:256].zero_()                       # the error word only: flags stay as the timeout left them
    note("check_flags: call over leftover flags, ll_max=%d" % ll_max)
    rc.all_reduce(src, empty_ranks(P, n, "f32"), ws=ws)
    assert rc.last_error(ws)[0] == N.RING_EPROTOCOL
    rc.workspace_init(ws)
    dst = empty_ranks(P, n, "f32")
    rc.all_reduce(src, dst, ws=ws)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))

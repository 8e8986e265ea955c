"""GPU tests of the workspace's record of data left behind ("全归约 3：Ring——
每步大小恒定", edge cases: the signal rows of one call must not be read by
another).  Some calls leave data in their workspace (bf16 partial sums of the
flag rounds, circulating-psum slots, partial GEMM tiles); a later call whose
flags or low-latency words would lie over that data must report
RING_EWORKSPACE instead of reading it as set flags, while calls of one shape
and operation on one workspace never trip the check.  Every result that is
produced is compared with the oracle bit for bit."""
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


def _bf16_ranks(P, n, seed):
    return inputs.normal_bf16(P, n, seed=seed, std=1.0)


def _f32_ranks(P, n, seed):
    return inputs.normal_f32(P, n, seed=seed)


def test_other_shape_over_bf16_partial_sums_reports_eworkspace():
    """A bf16 all-reduce in the flag rounds (P = 4, 1 Mi per rank: 512 KiB
    chunks) leaves its fp32 partial sums in the workspace; an fp32 all-reduce
    of another shape (P = 8, 1 Mi per rank), whose flag table reaches into
    those partial sums, on the same uncleared workspace must end in
    RING_EWORKSPACE.  After a zero fill the same call gives the oracle's
    bits."""
    xa = _bf16_ranks(4, 1 << 20, 900)
    ws = rc.workspace(N.OP_ALL_REDUCE, 4, 1 << 20, torch.bfloat16)
    nb = rc.workspace_bytes(N.OP_ALL_REDUCE, 8, 1 << 20, torch.float32)
    assert nb <= ws.numel()
    note("ws record: bf16 all-reduce P=4 1Mi (flag rounds)")
    dst = empty_ranks(4, 1 << 20, "bf16")
    rc.all_reduce(to_dev(xa, "bf16"), dst, ws=ws)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(to_host(dst, "bf16"), oracle.all_reduce_bf16(xa))
    note("ws record: fp32 all-reduce P=8 1Mi over the partial sums")
    xb = _f32_ranks(8, 1 << 20, 901)
    src = to_dev(xb, "f32")
    dst = empty_ranks(8, 1 << 20, "f32")
    rc.all_reduce(src, dst, ws=ws)
    code, _ = rc.last_error(ws)
    assert code == N.RING_EWORKSPACE, code
    rc.workspace_init(ws)
    dst = empty_ranks(8, 1 << 20, "f32")
    rc.all_reduce(src, dst, ws=ws)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(xb)))


def test_same_shape_flag_then_low_latency_rounds():
    """The same bf16 shape in the flag rounds (low-latency rounds off) and
    then in the low-latency rounds, on one workspace sized for the latter,
    alternately: the flag rounds' partial sums never lie under the words of
    the low-latency rounds, and every call gives the oracle's bits."""
    P, n = 4, 4 * 4096
    x = _bf16_ranks(P, n, 902)
    want = oracle.all_reduce_bf16(x)
    src = to_dev(x, "bf16")
    ws = rc.workspace(N.OP_ALL_REDUCE, P, n, torch.bfloat16)
    for call, ll in enumerate((0, 262144, 0, 262144)):
        N.set_tuning(ll_max_chunk_bytes=ll)
        note("ws record: bf16 all-reduce P=%d n=%d call %d ll_max=%d" % (P, n, call, ll))
        dst = empty_ranks(P, n, "bf16")
        rc.all_reduce(src, dst, ws=ws)
        assert rc.last_error(ws)[0] == 0, call
        np.testing.assert_array_equal(to_host(dst, "bf16"), want, err_msg="call %d" % call)


@pytest.mark.parametrize("op", ["reduce_scatter", "all_reduce", "reduce_scatter_bidir", "psum"])
def test_repeated_calls_of_one_shape_never_trip(op):
    """Calls that leave data behind, repeated on one workspace: no error, the
    oracle's bits every time."""
    P, n = 4, 4 << 18                   # 512 KiB bf16 chunks: the flag rounds
    x = _bf16_ranks(P, n, 903)
    fn, ws_op, want = {
        "reduce_scatter": (rc.reduce_scatter, N.OP_REDUCE_SCATTER, oracle.reduce_scatter_bf16(x)[0]),
        "all_reduce": (rc.all_reduce, N.OP_ALL_REDUCE, oracle.all_reduce_bf16(x)),
        "reduce_scatter_bidir": (rc.reduce_scatter_bidir, N.OP_REDUCE_SCATTER_BIDIR,
                                 oracle.reduce_scatter_bidir_bf16(x)[0]),
        "psum": (rc.psum_circulating, N.OP_PSUM_CIRCULATING, oracle.psum_circulating_bf16(x)),
    }[op]
    C = n // P
    src = to_dev(x, "bf16")
    ws = rc.workspace(ws_op, P, n, torch.bfloat16)
    for call in range(3):
        note("ws record: %s bf16 P=%d call %d" % (op, P, call))
        dst = empty_ranks(P, n, "bf16")
        fn(src, dst, ws=ws)
        assert rc.last_error(ws)[0] == 0, call
        got = to_host(dst, "bf16")
        if op.startswith("reduce_scatter"):
            for r in range(P):
                np.testing.assert_array_equal(got[r, r * C:(r + 1) * C], want[r, r * C:(r + 1) * C])
        else:
            np.testing.assert_array_equal(got, want)


def test_psum_slots_then_larger_flag_table_reports_eworkspace():
    """The circulating psum leaves its receive slots in the workspace; a
    ring all-reduce whose flag table reaches them reports RING_EWORKSPACE."""
    P, n = 4, 1 << 18
    x = _f32_ranks(P, n, 904)
    ws = rc.workspace(N.OP_PSUM_CIRCULATING, P, n, torch.float32)
    note("ws record: psum fp32 P=4")
    dst = empty_ranks(P, n, "f32")
    rc.psum_circulating(to_dev(x, "f32"), dst, ws=ws)
    assert rc.last_error(ws)[0] == 0
    xb = _f32_ranks(8, 1 << 20, 905)
    assert rc.workspace_bytes(N.OP_ALL_REDUCE, 8, 1 << 20, torch.float32) <= ws.numel()
    note("ws record: all-reduce P=8 over the slots")
    rc.all_reduce(to_dev(xb, "f32"), empty_ranks(8, 1 << 20, "f32"), ws=ws)
    assert rc.last_error(ws)[0] == N.RING_EWORKSPACE


def test_gemm_partial_tiles_then_ring_reports_eworkspace():
    """The fused GEMM + reduce-scatter leaves partial tiles in its workspace;
    a ring all-reduce whose flags reach them reports RING_EWORKSPACE, and
    after a zero fill gives the oracle's bits."""
    P, M, Nn, K = 2, 1024, 1024, 128
    rng = np.random.default_rng(906)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    a = [torch.from_numpy(A[q].view(np.int16)).cuda().view(torch.bfloat16) for q in range(P)]
    b = [torch.from_numpy(B[q].view(np.int16)).cuda().view(torch.bfloat16) for q in range(P)]
    out = [torch.empty((M // P, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    note("ws record: gemm_rs P=2 1024^2")
    ws = rc.gemm_reduce_scatter(a, b, out)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(np.stack([o.cpu().numpy() for o in out]), oracle.gemm_reduce_scatter(A, B))
    xb = _f32_ranks(8, 1 << 20, 907)
    assert rc.workspace_bytes(N.OP_ALL_REDUCE, 8, 1 << 20, torch.float32) <= ws.numel()
    src = to_dev(xb, "f32")
    note("ws record: all-reduce P=8 over the partial tiles")
    rc.all_reduce(src, empty_ranks(8, 1 << 20, "f32"), ws=ws)
    assert rc.last_error(ws)[0] == N.RING_EWORKSPACE
    rc.workspace_init(ws)
    dst = empty_ranks(8, 1 << 20, "f32")
    rc.all_reduce(src, dst, ws=ws)
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(xb)))


def test_side_stream_call_with_dropped_workspace():
    """A call on a side stream whose workspace the binding creates and the
    caller drops at once: the allocator must not hand that block out again
    while the side stream's kernel still uses it.  A tensor of the same size
    allocated and filled on the current stream right after keeps its fill,
    and the collective gives the oracle's bits."""
    P, n = 8, 8 << 20
    x = _f32_ranks(P, n, 908)
    src = to_dev(x, "f32")
    dst = empty_ranks(P, n, "f32")
    nb = max(rc.workspace_bytes(N.OP_ALL_REDUCE, P, n, torch.float32), 256)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    note("ws record: side-stream all-reduce with a dropped workspace")
    # keep the side stream busy first, so its collective is still pending
    # when the current stream reuses memory
    busy = torch.randn(4096, 4096, device="cuda")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(8):
            busy = busy @ busy * 1e-3
    rc.all_reduce(src, dst, stream=side)           # returned workspace dropped here
    fill = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")
    side.synchronize()
    torch.cuda.synchronize()
    assert bool((fill == 0xA5).all())
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))

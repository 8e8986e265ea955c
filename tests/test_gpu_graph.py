"""The collectives captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed.  Every entry point that computes is captured here.

The library allocates nothing, records no memset, and every kernel leaves
its flag table zeroed for the next call, so a captured call can be replayed
as often as an eager one.  Each graph here is replayed several times, with
the program's own eager work (input changes and eager calls of the library
on other buffers) and synchronisations between the replays, and every
replay is checked against the oracle or against the eager result: bit for
bit.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_collectives_amd import _native as N
from ring_collectives_amd import collectives as rc
from ring_collectives_amd import inputs

from _gpu_helpers import bits, empty_ranks, note, rs_written_chunks, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()
    yield


def _capture(fn):
    """Run fn eagerly once (kernels loaded, workspaces touched), then capture it."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_all_reduce_replays(kind):
    """P = 4 over 3 tiles and a ragged tail per chunk; between replays the
    inputs change and an eager all-reduce runs on other buffers with its own
    workspace."""
    P, n = 4, 4 * (3 * 4096 + 96)
    note("graph all_reduce %s" % kind)
    rng = np.random.default_rng(1300)
    x = rng.random((P, n), dtype=np.float32)
    if kind == "bf16":
        x = oracle.bf16_from_f32(x)
    dt = torch.float32 if kind == "f32" else torch.bfloat16
    src, dst = to_dev(x, kind), empty_ranks(P, n, kind)
    ws = rc.workspace(N.OP_ALL_REDUCE, P, n, dt)
    g = _capture(lambda: rc.all_reduce(src, dst, ws=ws))
    other_src, other_dst = to_dev(x[::-1].copy(), kind), empty_ranks(P, n, kind)
    other_ws = rc.workspace(N.OP_ALL_REDUCE, P, n, dt)
    ref = oracle.all_reduce if kind == "f32" else oracle.all_reduce_bf16
    for rep in range(3):
        for t in src:
            t.mul_(0.5)                                       # eager input change
        rc.all_reduce(other_src, other_dst, ws=other_ws)      # eager library call
        torch.cuda.synchronize()
        host_in = to_host(src, kind)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(ref(host_in)), err_msg="replay %d" % rep)
        np.testing.assert_array_equal(bits(to_host(other_dst, kind)), bits(ref(x[::-1].copy())))
    assert rc.last_error(ws)[0] == 0 and rc.last_error(other_ws)[0] == 0


def test_gemm_reduce_scatter_replays():
    """P = 4, 1024 x 256 x 128 on integer-valued operands (exact in any order)."""
    P, M, Nn, K = 4, 1024, 256, 128
    note("graph gemm_reduce_scatter")
    rng = np.random.default_rng(1310)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    dev = lambda a: [torch.from_numpy(np.ascontiguousarray(a[q]).view(np.int16)).cuda().view(torch.bfloat16)
                     for q in range(P)]
    a, b = dev(A), dev(B)
    out = [torch.empty((M // P, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws = rc.gemm_reduce_scatter(a, b, out)
    torch.cuda.synchronize()
    g = _capture(lambda: rc.gemm_reduce_scatter(a, b, out, ws=ws))
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))                             # eager: poison the output
        if rep:
            for t in a:
                t.neg_()                                      # eager input change (exact)
        torch.cuda.synchronize()
        A_now = np.stack([t.view(torch.int16).cpu().numpy().view(np.uint16) for t in a])
        g.replay()
        torch.cuda.synchronize()
        want = oracle.gemm_reduce_scatter(A_now, B)
        got = np.stack([o.cpu().numpy() for o in out])
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32), err_msg="replay %d" % rep)
    assert rc.last_error(ws)[0] == 0


@pytest.mark.parametrize("P,M,D,F", [(4, 256, 1024, 16384), (2, 1024, 256, 512)])
def test_mlp_layer_replays(P, M, D, F):
    """The chapter's shape (the unfused path: five launches) and a fused
    shape; each replay after an eager layer on the same weights with other
    activations, compared bit for bit with an eager run of the same inputs."""
    note("graph tp_mlp P=%d M=%d D=%d F=%d" % (P, M, D, F))
    x, w1, w2 = inputs.mlp_operands(P, M, D, F, seed=1320 + P)
    Mq, Fr = M // P, F // P
    dev = lambda a: [torch.from_numpy(np.ascontiguousarray(a[q]).view(np.int16)).cuda().view(torch.bfloat16)
                     for q in range(a.shape[0])]
    xs, W1, W2 = dev(x), dev(w1), dev(w2)
    full = [torch.empty((M, D), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    h = [torch.empty((M, Fr), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    out = [torch.empty((Mq, D), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    ws = rc.tp_mlp_workspace(P, M, D, F)
    g = _capture(lambda: rc.tp_mlp_layer(xs, W1, W2, full, h, out, ws=ws))
    xs2 = dev(x[::-1].copy())
    full2 = [torch.empty_like(t) for t in full]
    h2 = [torch.empty_like(t) for t in h]
    out2 = [torch.empty_like(t) for t in out]
    ws2 = rc.tp_mlp_workspace(P, M, D, F)
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))
        rc.tp_mlp_layer(xs2, W1, W2, full2, h2, out2, ws=ws2)   # eager layer, other activations
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in out] + [t.clone() for t in h]
        rc.tp_mlp_layer(xs, W1, W2, full, h, out, ws=ws2)        # eager, same inputs
        torch.cuda.synchronize()
        want = out + h
        for a_, b_ in zip(got, want):
            assert torch.equal(a_.view(torch.int16), b_.view(torch.int16)), "replay %d" % rep
    assert rc.last_error(ws)[0] == 0 and rc.last_error(ws2)[0] == 0


def _replays(g, change, eager, check, reps=3):
    """Replay g reps times; before each replay change the inputs and run
    eager library work (both eager), then check the replay's result."""
    for rep in range(reps):
        change(rep)
        eager()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check(rep)


def test_ppermute_replays():
    """P = 4 over 3 tiles and a ragged tail (fp32)."""
    P, n = 4, 3 * 4096 + 17
    note("graph ppermute")
    x = np.random.default_rng(1330).random((P, n), dtype=np.float32)
    src, dst = to_dev(x, "f32"), empty_ranks(P, n, "f32")
    other_src, other_dst = to_dev(x[::-1].copy(), "f32"), empty_ranks(P, n, "f32")
    g = _capture(lambda: rc.ppermute(src, dst))

    def change(rep):
        for t in src:
            t.mul_(0.5)
        for t in dst:
            t.fill_(float("nan"))

    def check(rep):
        np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.ppermute(to_host(src, "f32"))),
                                      err_msg="replay %d" % rep)
        np.testing.assert_array_equal(bits(to_host(other_dst, "f32")), bits(oracle.ppermute(x[::-1].copy())))

    _replays(g, change, lambda: rc.ppermute(other_src, other_dst), check)


@pytest.mark.parametrize("kind", ["f32", "i32"])
def test_reduce_scatter_replays(kind):
    """P = 4 over 3 tiles and a ragged tail per chunk: every chunk the
    reduce-scatter writes, against the oracle's ring order, bit for bit."""
    P, n = 4, 4 * (3 * 4096 + 96)
    C = n // P
    note("graph reduce_scatter %s" % kind)
    rng = np.random.default_rng(1340)
    x = (rng.random((P, n), dtype=np.float32) if kind == "f32"
         else rng.integers(-1000, 1000, size=(P, n), dtype=np.int32))
    dt = torch.float32 if kind == "f32" else torch.int32
    src, dst = to_dev(x, kind), empty_ranks(P, n, kind)
    ws = rc.workspace(N.OP_REDUCE_SCATTER, P, n, dt)
    other_src, other_dst = to_dev(x[::-1].copy(), kind), empty_ranks(P, n, kind)
    other_ws = rc.workspace(N.OP_REDUCE_SCATTER, P, n, dt)
    g = _capture(lambda: rc.reduce_scatter(src, dst, ws=ws))

    def change(rep):
        for t in src:
            if kind == "f32":
                t.mul_(0.5)
            else:
                t.neg_()

    def written(got, want, what):
        for r, c in rs_written_chunks(P):
            np.testing.assert_array_equal(bits(got[r, c * C:(c + 1) * C]), bits(want[r, c * C:(c + 1) * C]),
                                          err_msg="%s rank %d chunk %d" % (what, r, c))

    def check(rep):
        written(to_host(dst, kind), oracle.reduce_scatter(to_host(src, kind)), "replay %d" % rep)
        written(to_host(other_dst, kind), oracle.reduce_scatter(x[::-1].copy()), "eager")

    _replays(g, change, lambda: rc.reduce_scatter(other_src, other_dst, ws=other_ws), check)
    assert rc.last_error(ws)[0] == 0 and rc.last_error(other_ws)[0] == 0


def test_all_gather_replays():
    """P = 4, compact pieces of 2 tiles and a ragged tail (bf16)."""
    P, C = 4, 2 * 8192 + 40
    n = P * C
    note("graph all_gather")
    pieces = inputs.normal_bf16(P, C, seed=1350)
    src, dst = to_dev(pieces, "bf16"), empty_ranks(P, n, "bf16")
    ws = rc.workspace(N.OP_ALL_GATHER, P, n, torch.bfloat16)
    other_src, other_dst = to_dev(pieces[::-1].copy(), "bf16"), empty_ranks(P, n, "bf16")
    other_ws = rc.workspace(N.OP_ALL_GATHER, P, n, torch.bfloat16)
    g = _capture(lambda: rc.all_gather(dst, src=src, ws=ws))

    def change(rep):
        for t in src:
            t.neg_()
        for t in dst:
            t.view(torch.int16).fill_(0x7FC1)

    def check(rep):
        np.testing.assert_array_equal(to_host(dst, "bf16"), oracle.all_gather_pieces(to_host(src, "bf16")),
                                      err_msg="replay %d" % rep)
        np.testing.assert_array_equal(to_host(other_dst, "bf16"), oracle.all_gather_pieces(pieces[::-1].copy()))

    _replays(g, change, lambda: rc.all_gather(other_dst, src=other_src, ws=other_ws), check)
    assert rc.last_error(ws)[0] == 0 and rc.last_error(other_ws)[0] == 0


@pytest.mark.parametrize("op", ["bidir", "psum"])
def test_bidir_and_psum_replays(op):
    """The bidirectional reduce-scatter and the circulating psum, P = 4,
    fp32 chunks of 2 tiles and a ragged tail."""
    P, n = 4, 4 * (2 * 4096 + 24)
    note("graph %s" % op)
    x = inputs.normal_f32(P, n, seed=1360)
    run = rc.reduce_scatter_bidir if op == "bidir" else rc.psum_circulating
    code = N.OP_REDUCE_SCATTER_BIDIR if op == "bidir" else N.OP_PSUM_CIRCULATING
    ref = oracle.reduce_scatter_bidir if op == "bidir" else (lambda v: oracle.psum_circulating(v)[0])
    src, dst = to_dev(x, "f32"), empty_ranks(P, n, "f32")
    ws = rc.workspace(code, P, n, torch.float32)
    other_src, other_dst = to_dev(x[::-1].copy(), "f32"), empty_ranks(P, n, "f32")
    other_ws = rc.workspace(code, P, n, torch.float32)
    g = _capture(lambda: run(src, dst, ws=ws))

    def change(rep):
        for t in src:
            t.mul_(-0.5)
        for t in dst:
            t.fill_(float("nan"))

    def check(rep):
        np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(ref(to_host(src, "f32"))),
                                      err_msg="replay %d" % rep)
        np.testing.assert_array_equal(bits(to_host(other_dst, "f32")), bits(ref(x[::-1].copy())))

    _replays(g, change, lambda: run(other_src, other_dst, ws=other_ws), check)
    assert rc.last_error(ws)[0] == 0 and rc.last_error(other_ws)[0] == 0


@pytest.mark.parametrize("tile", [128, 256])
def test_all_gather_gemm_replays(tile):
    """P = 4, 1024 x 512 x 128 on integer-valued operands (exact in any
    order): the gathered A and C of every replay, bit for bit; the panel
    flags the last workgroup clears must be clear again for each replay."""
    P, M, Nn, K = 4, 1024, 512, 128
    note("graph all_gather_gemm tile %d" % tile)
    old = N.get_tuning()
    N.set_tuning(gemm_tile_n=tile)
    try:
        rng = np.random.default_rng(1370)
        As = inputs.small_int_bf16(rng, (P, M // P, K))
        B = inputs.small_int_bf16(rng, (P, K, Nn))
        dev = lambda a: [torch.from_numpy(np.ascontiguousarray(a[q]).view(np.int16)).cuda().view(torch.bfloat16)
                         for q in range(P)]
        a, b = dev(As), dev(B)
        full = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
        C = [torch.empty((M, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
        ws = rc.all_gather_gemm(a, b, full, C)
        torch.cuda.synchronize()
        other_a = dev(As[::-1].copy())
        other_full = [torch.empty_like(t) for t in full]
        other_C = [torch.empty_like(t) for t in C]
        other_ws = rc.all_gather_gemm(other_a, b, other_full, other_C)
        torch.cuda.synchronize()
        g = _capture(lambda: rc.all_gather_gemm(a, b, full, C, ws=ws))

        def change(rep):
            for t in a:
                t.neg_()
            for t in C:
                t.fill_(float("nan"))
            for t in full:
                t.view(torch.int16).fill_(0x7FC1)

        def host(ts):
            return np.stack([t.view(torch.int16).cpu().numpy().view(np.uint16) for t in ts])

        def check(rep):
            want_full, want_c = oracle.all_gather_gemm(host(a), B)
            np.testing.assert_array_equal(host(full), want_full, err_msg="replay %d" % rep)
            got_c = np.stack([t.cpu().numpy() for t in C])
            np.testing.assert_array_equal(got_c.view(np.uint32), want_c.view(np.uint32), err_msg="replay %d" % rep)
            _, other_c = oracle.all_gather_gemm(As[::-1].copy(), B)
            np.testing.assert_array_equal(np.stack([t.cpu().numpy() for t in other_C]).view(np.uint32),
                                          other_c.view(np.uint32))

        _replays(g, change, lambda: rc.all_gather_gemm(other_a, b, other_full, other_C, ws=other_ws), check)
        assert rc.last_error(ws)[0] == 0 and rc.last_error(other_ws)[0] == 0
    finally:
        N.set_tuning(**old)

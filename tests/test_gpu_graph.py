"""The collectives captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed.

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

from _gpu_helpers import bits, empty_ranks, note, to_dev, to_host

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

"""The low-latency rounds of the one-way ring collectives against the oracle
and against the flag rounds, bit for bit, through the C ABI.

In the low-latency rounds every value a rank passes right travels in an
8-byte word with its ready mark; the neighbour polls the word itself and
clears it.  Every case here runs on the same inputs with
ll_max_chunk_bytes at its default (chunks of at most 256 KiB take those
rounds) and at 0 (the per-tile flag rounds), and both must give the oracle's
bits: the same chunks, the same additions in the same order.  After a call
that took the low-latency rounds the whole workspace is zero again (the
status word, the untouched flags, every word cleared by its reader), which
is what lets the next call, or a graph replay, start from it.  Chunks of
1000 elements leave a ragged last tile position of 232 elements.
"""
import numpy as np
import pytest
import torch

import oracle
from ring_collectives_amd import _native as N
from ring_collectives_amd import collectives as rc

from _gpu_helpers import bits, empty_ranks, note, rs_written_chunks, to_dev, to_host

pytestmark = pytest.mark.gpu

MODES = {"ll": 256 << 10, "flags": 0}
DT = {"f32": torch.float32, "i32": torch.int32, "bf16": torch.bfloat16}


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


def _data(kind, P, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "f32":
        return rng.random((P, n), dtype=np.float32)
    if kind == "i32":
        return rng.integers(-1000, 1000, size=(P, n), endpoint=True, dtype=np.int32)
    return oracle.bf16_from_f32(rng.standard_normal((P, n), dtype=np.float32))


def _ws_clean(ws):
    torch.cuda.synchronize()
    return int(torch.count_nonzero(ws).item()) == 0


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("kind", ["f32", "i32", "bf16"])
@pytest.mark.parametrize("P,C", [(2, 1000), (3, 1000), (4, 4096), (8, 1000), (16, 256)])
@pytest.mark.parametrize("in_place", [False, True])
def test_all_reduce(P, C, kind, mode, in_place):
    note("ll all_reduce P=%d C=%d %s %s in_place=%s" % (P, C, kind, mode, in_place))
    N.set_tuning(ll_max_chunk_bytes=MODES[mode])
    x = _data(kind, P, P * C, 900 + P)
    src = to_dev(x, kind)
    dst = src if in_place else empty_ranks(P, P * C, kind)
    ws = rc.workspace(N.OP_ALL_REDUCE, P, P * C, DT[kind])
    rc.all_reduce(src, dst, ws=ws)
    assert rc.last_error(ws) == (0, 0)
    want = oracle.all_reduce_bf16(x) if kind == "bf16" else oracle.all_reduce(x)
    np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(want))
    if mode == "ll":
        assert _ws_clean(ws)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("kind", ["f32", "i32", "bf16"])
@pytest.mark.parametrize("P", [2, 3, 5, 8])
def test_reduce_scatter(P, kind, mode):
    """fp32 / int32: every chunk the ring writes holds the oracle's partial
    sum; bf16: the owners' chunks (its partial sums travel in the words or
    the carry, not in dst)."""
    note("ll reduce_scatter P=%d %s %s" % (P, kind, mode))
    N.set_tuning(ll_max_chunk_bytes=MODES[mode])
    C = 1000
    x = _data(kind, P, P * C, 910 + P)
    src = to_dev(x, kind)
    dst = empty_ranks(P, P * C, kind)
    ws = rc.workspace(N.OP_REDUCE_SCATTER, P, P * C, DT[kind])
    rc.reduce_scatter(src, dst, ws=ws)
    assert rc.last_error(ws) == (0, 0)
    got = to_host(dst, kind)
    if kind == "bf16":
        want, _ = oracle.reduce_scatter_bf16(x)
        pairs = [(r, r) for r in range(P)]
    else:
        want = oracle.reduce_scatter(x)
        pairs = rs_written_chunks(P)
    for r, c in pairs:
        np.testing.assert_array_equal(bits(got[r, c * C:(c + 1) * C]), bits(want[r, c * C:(c + 1) * C]),
                                      err_msg="rank %d chunk %d" % (r, c))
    if mode == "ll":
        assert _ws_clean(ws)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("kind", ["f32", "i32", "bf16"])
@pytest.mark.parametrize("P", [2, 4, 7])
@pytest.mark.parametrize("compact", [False, True])
def test_all_gather(P, kind, mode, compact):
    note("ll all_gather P=%d %s %s compact=%s" % (P, kind, mode, compact))
    N.set_tuning(ll_max_chunk_bytes=MODES[mode])
    C = 1000
    x = _data(kind, P, P * C, 920 + P)
    pieces = np.stack([x[r, r * C:(r + 1) * C] for r in range(P)])
    dst = empty_ranks(P, P * C, kind)
    ws = rc.workspace(N.OP_ALL_GATHER, P, P * C, DT[kind])
    if compact:
        rc.all_gather(dst, src=to_dev(pieces, kind), ws=ws)
    else:
        for r, t in enumerate(to_dev(pieces, kind)):
            dst[r][r * C:(r + 1) * C].copy_(t)
        rc.all_gather(dst, ws=ws)
    assert rc.last_error(ws) == (0, 0)
    np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(oracle.all_gather_pieces(pieces)))
    if mode == "ll":
        assert _ws_clean(ws)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_sixty_four_ranks(mode):
    """126 rounds, 256 elements per chunk: one tile position per chunk."""
    note("ll all_reduce P=64 %s" % mode)
    N.set_tuning(ll_max_chunk_bytes=MODES[mode])
    P, C = 64, 256
    x = _data("f32", P, P * C, 930)
    src, dst = to_dev(x, "f32"), empty_ranks(P, P * C, "f32")
    ws = rc.workspace(N.OP_ALL_REDUCE, P, P * C, torch.float32)
    rc.all_reduce(src, dst, ws=ws)
    assert rc.last_error(ws) == (0, 0)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))


def test_one_workspace_many_calls():
    """Calls of different collectives, dtypes and sizes share one workspace,
    alternating between the two kinds of rounds; each call's result is the
    oracle's and the workspace ends clean."""
    P, C = 4, 4096
    ws = rc.workspace(N.OP_ALL_REDUCE, P, P * C, torch.bfloat16)
    cases = [("ar", "f32", 1000, "ll"), ("rs", "i32", 4096, "flags"), ("ar", "bf16", 4096, "ll"),
             ("ag", "f32", 256, "ll"), ("ar", "i32", 1000, "flags"), ("ar", "f32", 4096, "ll"),
             ("rs", "f32", 1000, "ll")]
    for i, (op, kind, c, mode) in enumerate(cases):
        note("ll shared workspace call %d: %s %s C=%d %s" % (i, op, kind, c, mode))
        N.set_tuning(ll_max_chunk_bytes=MODES[mode])
        x = _data(kind, P, P * c, 940 + i)
        dst = empty_ranks(P, P * c, kind)
        if op == "ar":
            rc.all_reduce(to_dev(x, kind), dst, ws=ws)
            want = oracle.all_reduce_bf16(x) if kind == "bf16" else oracle.all_reduce(x)
            np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(want), err_msg="call %d" % i)
        elif op == "rs":
            rc.reduce_scatter(to_dev(x, kind), dst, ws=ws)
            got, want = to_host(dst, kind), oracle.reduce_scatter(x)
            for r in range(P):
                np.testing.assert_array_equal(bits(got[r, r * c:(r + 1) * c]), bits(want[r, r * c:(r + 1) * c]))
        else:
            pieces = np.stack([x[r, r * c:(r + 1) * c] for r in range(P)])
            rc.all_gather(dst, src=to_dev(pieces, kind), ws=ws)
            np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(oracle.all_gather_pieces(pieces)))
        assert rc.last_error(ws) == (0, 0)
    assert _ws_clean(ws)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_watchdog_in_both_forms(mode):
    """Rank 0 never passes on round 1's values (or flags): rank 1's wait in
    round 2, or a wait further down the broken chain, ends in RING_ETIMEOUT;
    after a re-initialisation the same workspace gives the right sums."""
    note("ll watchdog drop_round=2 %s" % mode)
    P, C = 4, 4096
    x = _data("f32", P, P * C, 950)
    src, dst = to_dev(x, "f32"), empty_ranks(P, P * C, "f32")
    ws = rc.workspace(N.OP_ALL_REDUCE, P, P * C, torch.float32)
    N.set_tuning(ll_max_chunk_bytes=MODES[mode], drop_round=2, timeout_s=0.05)
    rc.all_reduce(src, dst, ws=ws)
    code, info = rc.last_error(ws)
    assert code == N.RING_ETIMEOUT
    rank, rnd = info & 0xFF, (info >> 8) & 0xFF
    assert 2 <= rnd <= 2 * P - 3 and (rank - 1) % P == (rnd - 2) % P, (rank, rnd)
    N.set_tuning(drop_round=0, timeout_s=5.0)
    rc.workspace_init(ws)
    rc.all_reduce(src, dst, ws=ws)
    assert rc.last_error(ws) == (0, 0)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))


def test_mlp_layer_both_forms_agree():
    """The MLP layer at the chapter's shape (its all-gather and its fp32
    reduce-scatter with the bf16 result both take the low-latency rounds by
    default) gives the same bits with the flag rounds."""
    from ring_collectives_amd import inputs
    P, M, D, F = 4, 256, 1024, 16384
    note("ll tp_mlp P=%d M=%d both forms" % (P, M))
    x, w1, w2 = inputs.mlp_operands(P, M, D, F, seed=960)
    dev = lambda a: [torch.from_numpy(np.ascontiguousarray(a[q]).view(np.int16)).cuda().view(torch.bfloat16)
                     for q in range(a.shape[0])]
    xs, W1, W2 = dev(x), dev(w1), dev(w2)
    res = {}
    for mode in ("ll", "flags"):
        N.set_tuning(ll_max_chunk_bytes=MODES[mode])
        full = [torch.empty((M, D), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
        h = [torch.empty((M, F // P), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
        out = [torch.full((M // P, D), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
        ws = rc.tp_mlp_workspace(P, M, D, F)
        rc.tp_mlp_layer(xs, W1, W2, full, h, out, ws=ws)
        assert rc.last_error(ws) == (0, 0)
        res[mode] = [t.view(torch.int16).cpu() for t in out + full]
    for a, b in zip(res["ll"], res["flags"]):
        assert torch.equal(a, b)

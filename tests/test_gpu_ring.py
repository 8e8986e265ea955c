"""GPU parity of the ring collectives against the CPU oracle, element by
element on the same seeded inputs, through the C ABI.

Bar: bit-exact for int32, bf16 and fp32 (the HIP path adds in the same order
as the oracle); plus the fp32/bf16 tolerances against the fp64 rank-order sum
(componentwise, normalised by sum |x|: 1e-6 P for fp32, 1e-2 for bf16).
"""
import numpy as np
import pytest
import torch

import oracle
from ring_collectives_amd import _native as N
from ring_collectives_amd import collectives as rc
from ring_collectives_amd import inputs

from _gpu_helpers import (bits, empty_ranks, note, poison_like, rs_written_chunks, to_dev,
                          to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()   # fail loudly if the library is missing
    yield


@pytest.fixture(autouse=True)
def _default_tuning():
    old = N.get_tuning()
    yield
    N.set_tuning(**old)


def _run_ar(x, kind, in_place=False, ws=None):
    src = to_dev(x, kind)
    dst = src if in_place else empty_ranks(x.shape[0], x.shape[1], kind)
    rc.all_reduce(src, dst, ws=ws)
    return to_host(dst, kind)


# ---------------------------------------------------------------- ppermute
@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("kind", ["f32", "i32", "bf16"])
def test_ppermute(P, kind):
    note("ppermute P=%d %s" % (P, kind))
    rng = np.random.default_rng(100 + P)
    if kind == "f32":
        x = inputs.to_chunk_major(inputs.small_f32(P, (8, 512)), P) if 512 % P == 0 else \
            rng.random((P, 4096), dtype=np.float32)
    elif kind == "i32":
        x = inputs.to_chunk_major(inputs.ring_i32(P), P)
    else:
        x = inputs.normal_bf16(P, 4096 + 8, seed=3)
    src = to_dev(x, kind)
    dst = empty_ranks(P, x.shape[1], kind)
    rc.ppermute(src, dst)
    np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(oracle.ppermute(x)))


@pytest.mark.parametrize("n", [1, 3, 1001, (1 << 20) + 7])
def test_ppermute_ragged(n):
    note("ppermute ragged n=%d" % n)
    x = np.random.default_rng(n).integers(-2**31, 2**31 - 1, size=(4, n), dtype=np.int32)
    src = to_dev(x, "i32")
    dst = empty_ranks(4, n, "i32")
    rc.ppermute(src, dst)
    np.testing.assert_array_equal(to_host(dst, "i32"), oracle.ppermute(x))


# ---------------------------------------------------------------- int32 RS / AG (cfg2)
@pytest.mark.parametrize("P", [2, 3, 4, 8])
def test_reduce_scatter_int32(P):
    note("reduce_scatter int32 P=%d" % P)
    x = inputs.to_chunk_major(inputs.ring_i32(P), P)
    src = to_dev(x, "i32")
    dst = empty_ranks(P, x.shape[1], "i32")
    rc.reduce_scatter(src, dst)
    got = to_host(dst, "i32")
    want = oracle.reduce_scatter(x)
    C = x.shape[1] // P
    for r, c in rs_written_chunks(P):
        np.testing.assert_array_equal(got[r, c * C:(c + 1) * C], want[r, c * C:(c + 1) * C],
                                      err_msg="rank %d chunk %d" % (r, c))
    # owner chunks against the plain sum over ranks
    total = x.astype(np.int64).sum(axis=0)
    for r in range(P):
        np.testing.assert_array_equal(got[r, r * C:(r + 1) * C], total[r * C:(r + 1) * C])


@pytest.mark.parametrize("P", [2, 3, 4, 8])
@pytest.mark.parametrize("compact", [True, False])
def test_all_gather_int32(P, compact):
    note("all_gather int32 P=%d compact=%s" % (P, compact))
    x = inputs.to_chunk_major(inputs.ring_i32(P), P)
    C = x.shape[1] // P
    pieces = np.stack([x[r, r * C:(r + 1) * C] for r in range(P)])
    dst = empty_ranks(P, x.shape[1], "i32")
    if compact:
        rc.all_gather(dst, src=to_dev(pieces, "i32"))
    else:
        for r in range(P):
            dst[r][r * C:(r + 1) * C].copy_(torch.from_numpy(pieces[r]).cuda())
        rc.all_gather(dst)
    got = to_host(dst, "i32")
    want = oracle.all_gather_pieces(pieces)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("P", [2, 4, 8])
def test_all_gather_bf16_f32_compact(P):
    note("all_gather bf16/f32 P=%d" % P)
    for kind, x in (("bf16", inputs.normal_bf16(P, 8 * 1000 * P, seed=21)),
                    ("f32", inputs.normal_f32(P, 1000 * P, seed=22))):
        C = x.shape[1] // P
        pieces = np.stack([x[r, r * C:(r + 1) * C] for r in range(P)])
        dst = empty_ranks(P, x.shape[1], kind)
        rc.all_gather(dst, src=to_dev(pieces, kind))
        np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(oracle.all_gather_pieces(pieces)))


# ---------------------------------------------------------------- fp32 all-reduce
@pytest.mark.parametrize("P", [2, 4])
def test_all_reduce_small_f32(P):
    """Small fp32 ring: (8, 512) per rank, uniform [0, 1), seed 0."""
    note("all_reduce small f32 P=%d" % P)
    x = inputs.to_chunk_major(inputs.small_f32(P, (8, 512)), P)
    got = _run_ar(x, "f32")
    np.testing.assert_array_equal(bits(got), bits(oracle.all_reduce(x)))


@pytest.mark.parametrize("P", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("C", [1, 7, 2048 * 3 + 100, 2048 * 5])
def test_all_reduce_sizes_f32(P, C):
    """Ragged chunk sizes (not a multiple of the vector width or the tile)."""
    note("all_reduce f32 P=%d C=%d" % (P, C))
    x = inputs.normal_f32(P, P * C, seed=30 + C % 97)
    got = _run_ar(x, "f32")
    np.testing.assert_array_equal(bits(got), bits(oracle.all_reduce(x)))


@pytest.mark.parametrize("P", [2, 4, 8])
def test_all_reduce_in_place(P):
    note("all_reduce in place P=%d" % P)
    x = inputs.normal_f32(P, P * 12345 * 4, seed=40)
    got = _run_ar(x, "f32", in_place=True)
    np.testing.assert_array_equal(bits(got), bits(oracle.all_reduce(x)))


@pytest.mark.parametrize("P", [2, 8])
def test_reduce_scatter_in_place_f32(P):
    note("reduce_scatter in place P=%d" % P)
    x = inputs.normal_f32(P, P * 20000, seed=41)
    t = to_dev(x, "f32")
    rc.reduce_scatter(t, t)
    got = to_host(t, "f32")
    want = oracle.reduce_scatter(x)
    np.testing.assert_array_equal(bits(got), bits(want))   # in place: every chunk defined


@pytest.mark.parametrize("P", [2, 4, 8])
def test_all_reduce_int32(P):
    note("all_reduce int32 P=%d" % P)
    x = inputs.to_chunk_major(inputs.ring_i32(P, width_per_rank=1000), P)
    got = _run_ar(x, "i32")
    np.testing.assert_array_equal(got, oracle.all_reduce(x))


def test_int32_wraps():
    note("all_reduce int32 wrap")
    P = 4
    x = np.full((P, P * 4096), 2**31 - 1, dtype=np.int32)
    got = _run_ar(x, "i32")
    np.testing.assert_array_equal(got, oracle.all_reduce(x))


def test_repeated_calls_reuse_workspace():
    """The flag table clears itself: back-to-back calls on one workspace,
    with different data and sizes, stay exact."""
    P = 8
    n_big = P * 2048 * 40
    ws = rc.workspace(N.OP_ALL_REDUCE, P, n_big, torch.float32)
    for i, n in enumerate([n_big, P * 777, n_big, P * 2048 * 3]):
        note("repeated all_reduce call %d n=%d" % (i, n))
        x = inputs.normal_f32(P, n, seed=50 + i)
        got = _run_ar(x, "f32", ws=ws)
        np.testing.assert_array_equal(bits(got), bits(oracle.all_reduce(x)))
        assert rc.last_error(ws) == (0, 0)


@pytest.mark.parametrize("tile_vecs", [4, 8, 16])
@pytest.mark.parametrize("map_mode", [0, 2])
def test_tuning_does_not_change_bits(tile_vecs, map_mode):
    P = 8
    x = inputs.normal_f32(P, P * (64 * 16 * 4 * 9 + 44), seed=60)
    want = oracle.all_reduce(x)
    for wpc in (4, 8, 16):
        note("tuning tile_vecs=%d map=%d waves_per_cu=%d" % (tile_vecs, map_mode, wpc))
        N.set_tuning(tile_vecs=tile_vecs, map_mode=map_mode, waves_per_cu=wpc)
        np.testing.assert_array_equal(bits(_run_ar(x, "f32")), bits(want))


def test_stepwise_debug_mode_matches():
    """One launch per round (stream order instead of flags) gives the same
    bits as the flag-synchronised launch."""
    P = 8
    x = inputs.normal_f32(P, P * 50000, seed=61)
    note("stepwise all_reduce")
    N.set_tuning(stepwise=1)
    a = _run_ar(x, "f32")
    N.set_tuning(stepwise=0)
    b = _run_ar(x, "f32")
    np.testing.assert_array_equal(bits(a), bits(b))
    np.testing.assert_array_equal(bits(a), bits(oracle.all_reduce(x)))


def test_few_waves_many_tiles():
    """Minimum waves per CU and small tiles: every wave walks many tiles."""
    P = 16
    N.set_tuning(tile_vecs=4, waves_per_cu=4)
    x = inputs.normal_f32(P, P * 1024 * 600, seed=62)
    note("few waves many tiles")
    np.testing.assert_array_equal(bits(_run_ar(x, "f32")), bits(oracle.all_reduce(x)))


# ---------------------------------------------------------------- bf16
@pytest.mark.parametrize("P", [2, 3, 4, 16])
@pytest.mark.parametrize("C", [8, 2048 * 2 + 24, 4096 * 3])
def test_all_reduce_bf16(P, C):
    note("all_reduce bf16 P=%d C=%d" % (P, C))
    x = inputs.normal_bf16(P, P * C, seed=70 + P)
    got = _run_ar(x, "bf16")
    np.testing.assert_array_equal(got, oracle.all_reduce_bf16(x))


def test_all_reduce_bf16_unaligned_chunks():
    P, C = 4, 1001     # chunk starts not 16-byte aligned: scalar path
    note("all_reduce bf16 unaligned")
    x = inputs.normal_bf16(P, P * C, seed=71)
    np.testing.assert_array_equal(_run_ar(x, "bf16"), oracle.all_reduce_bf16(x))


@pytest.mark.parametrize("P", [2, 4, 16])
def test_reduce_scatter_bf16(P):
    note("reduce_scatter bf16 P=%d" % P)
    x = inputs.normal_bf16(P, P * 4096 * 2, seed=72)
    src = to_dev(x, "bf16")
    dst = empty_ranks(P, x.shape[1], "bf16")
    rc.reduce_scatter(src, dst)
    got = to_host(dst, "bf16")
    want, _ = oracle.reduce_scatter_bf16(x)
    C = x.shape[1] // P
    for r in range(P):
        np.testing.assert_array_equal(got[r, r * C:(r + 1) * C], want[r, r * C:(r + 1) * C])


# ---------------------------------------------------------------- errors
def test_workspace_too_small_raises():
    P = 4
    x = to_dev(inputs.normal_f32(P, P * 4096, seed=80), "f32")
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(N.RingError) as e:
        rc.all_reduce(x, x, ws=small)
    assert e.value.code == N.RING_EWORKSPACE


def test_watchdog_reports_timeout():
    """Rank 0 is told never to signal round 2: its right neighbour's bounded
    wait ends in RING_ETIMEOUT and every wave exits.  The first wave to give
    up is on the broken chain: rank 1 at round 2, or a rank further right
    waiting for the round after (rank 1 + i at round 2 + i)."""
    P = 4
    x = inputs.normal_f32(P, P * 4096 * 4, seed=81)
    src = to_dev(x, "f32")
    dst = empty_ranks(P, x.shape[1], "f32")
    ws = rc.workspace(N.OP_ALL_REDUCE, P, x.shape[1], torch.float32)
    note("watchdog drop_round=2")
    N.set_tuning(drop_round=2, timeout_s=0.05)
    rc.all_reduce(src, dst, ws=ws)
    code, info = rc.last_error(ws)
    assert code == N.RING_ETIMEOUT
    rank, rnd = info & 0xFF, (info >> 8) & 0xFF
    assert 2 <= rnd <= 2 * P - 3 and (rank - 1) % P == (rnd - 2) % P, (rank, rnd)
    # re-initialise the workspace and run normally
    N.set_tuning(drop_round=0, timeout_s=5.0)
    rc.workspace_init(ws)
    rc.all_reduce(src, dst, ws=ws)
    assert rc.last_error(ws) == (0, 0)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))


# ---------------------------------------------------------------- full sizes
def test_full_size_fp32_p8_64Mi():
    """The bandwidth workload (P = 8, 64 Mi fp32 per rank, normal(0, 1), seed
    2) in the default launch configuration: every element bit for bit, plus
    the componentwise bound against the fp64 rank-order sum on a sample."""
    P, n = 8, 64 << 20
    note("full size fp32 P=8 generate")
    x = inputs.normal_f32(P, n, seed=inputs.SEED_F32_BW)
    note("full size fp32 P=8 run")
    got = _run_ar(x, "f32")
    want = oracle.all_reduce(x)
    np.testing.assert_array_equal(bits(got), bits(want))
    idx = np.random.default_rng(0).integers(0, n, size=1 << 16)
    ref, mag = oracle.rank_sum_f64(np.ascontiguousarray(x[:, idx]))
    err = np.abs(got[0, idx].astype(np.float64) - ref) / mag
    assert err.max() <= 1e-6 * P


def test_full_size_bf16_p16_128Mi():
    """The gradient-bucket workload (P = 16, 128 Mi bf16 per rank,
    normal(0, 0.01), seed 3): every element bit for bit against the oracle's
    fp32-carry ring, and within 1e-2 of the fp64 sum on a sample."""
    P, n = 16, 128 << 20
    note("full size bf16 P=16 generate")
    x = inputs.normal_bf16(P, n, seed=inputs.SEED_BF16)
    note("full size bf16 P=16 run")
    got = _run_ar(x, "bf16")
    want = oracle.all_reduce_bf16(x)
    np.testing.assert_array_equal(got, want)
    idx = np.random.default_rng(1).integers(0, n, size=1 << 16)
    ref, mag = oracle.rank_sum_f64(np.ascontiguousarray(x[:, idx]), bf16=True)
    err = np.abs(oracle.bf16_to_f32(got[0, idx]).astype(np.float64) - ref) / mag
    assert err.max() <= 1e-2


# ---------------------------------------------------------------- more ranks
@pytest.mark.parametrize("P,C", [(6, 2048 * 3 + 40), (7, 1001), (12, 4096 + 8), (32, 520), (64, 100)])
@pytest.mark.parametrize("kind", ["f32", "i32", "bf16"])
@pytest.mark.parametrize("ll", [256 << 10, 0])
def test_more_ranks_every_collective(P, C, kind, ll):
    """Rank counts 6, 7, 12, 32 and 64 (the library's maximum), ragged
    chunks: ppermute, reduce-scatter (each owner's chunk), all-gather,
    all-reduce, the bidirectional reduce-scatter and the circulating psum,
    every bit against the oracle; the one-way collectives in both the
    low-latency rounds (chunks this small take them by default) and the flag
    rounds."""
    note("more ranks P=%d C=%d %s ll=%d" % (P, C, kind, ll))
    N.set_tuning(ll_max_chunk_bytes=ll)
    n = P * C
    rng = np.random.default_rng(1500 + P)
    if kind == "i32":
        x = rng.integers(-1000, 1000, size=(P, n), endpoint=True, dtype=np.int32)
    elif kind == "f32":
        x = rng.standard_normal((P, n), dtype=np.float32)
    else:
        x = oracle.bf16_from_f32((rng.standard_normal((P, n)) * 0.01).astype(np.float32))
    dt = {"f32": torch.float32, "i32": torch.int32, "bf16": torch.bfloat16}[kind]
    ws = rc.workspace(N.OP_REDUCE_SCATTER_BIDIR, P, n, dt)    # the ring calls, one after the other
    ws_psum = rc.workspace(N.OP_PSUM_CIRCULATING, P, n, dt)
    src = to_dev(x, kind)

    dst = empty_ranks(P, n, kind)
    rc.ppermute(src, dst)
    np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(oracle.ppermute(x)))

    ar = oracle.all_reduce_bf16(x) if kind == "bf16" else oracle.all_reduce(x)
    dst = empty_ranks(P, n, kind)
    rc.all_reduce(src, dst, ws=ws)
    np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(ar))

    for name, fn in (("reduce_scatter", rc.reduce_scatter), ("bidir", rc.reduce_scatter_bidir)):
        dst = empty_ranks(P, n, kind)
        fn(src, dst, ws=ws)
        got = to_host(dst, kind)
        if kind == "bf16":
            want = (oracle.reduce_scatter_bf16(x)[0] if name == "reduce_scatter"
                    else oracle.reduce_scatter_bidir_bf16(x)[0])
        else:
            want = oracle.reduce_scatter(x) if name == "reduce_scatter" else oracle.reduce_scatter_bidir(x)
        for r in range(P):
            np.testing.assert_array_equal(bits(got[r, r * C:(r + 1) * C]), bits(want[r, r * C:(r + 1) * C]),
                                          err_msg="%s rank %d" % (name, r))

    state = np.stack([x[r] for r in range(P)])
    dst = to_dev(state, kind)
    rc.all_gather(dst, ws=ws)
    np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(oracle.all_gather(state)))

    dst = empty_ranks(P, n, kind)
    rc.psum_circulating(src, dst, ws=ws_psum)
    want = oracle.psum_circulating_bf16(x) if kind == "bf16" else oracle.psum_circulating(x)[0]
    np.testing.assert_array_equal(bits(to_host(dst, kind)), bits(want))
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0 and rc.last_error(ws_psum)[0] == 0


def test_side_stream_with_a_fresh_workspace():
    """A call on a stream other than torch's current one, with no workspace
    given: the binding zero-fills one on the current stream and makes the
    call's stream wait for it; the result is the oracle's."""
    note("side stream, fresh workspace")
    P = 4
    x = inputs.to_chunk_major(inputs.small_f32(P, (8, 512)), P)
    src = to_dev(x, "f32")
    dst = empty_ranks(P, x.shape[1], "f32")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ws = rc.all_reduce(src, dst, stream=side)
    side.synchronize()
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))
    assert rc.last_error(ws, stream=side)[0] == 0


def test_ring_calls_overlap_compute_on_other_streams():
    """Ring calls on side streams while a chain of vendor GEMMs occupies the
    main stream.  The ring kernels' waits stay within a tile position's ring
    of P consecutive waves, so every prefix of a launch's dispatch order
    holds complete rings and a call progresses with only part of its grid
    resident: the all-reduce, the bidirectional reduce-scatter and the
    circulating psum, each on its own stream, must give the oracle's bits
    and no watchdog error while the GEMMs run."""
    P, n = 8, 8 * (1 << 20)
    note("ring calls beside GEMMs on other streams")
    x = inputs.normal_f32(P, n, seed=1380)
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    calls = [(rc.all_reduce, N.OP_ALL_REDUCE, oracle.all_reduce),
             (rc.reduce_scatter_bidir, N.OP_REDUCE_SCATTER_BIDIR, oracle.reduce_scatter_bidir),
             (rc.psum_circulating, N.OP_PSUM_CIRCULATING, lambda v: oracle.psum_circulating(v)[0])]
    runs = []
    for fn, op, ref in calls:
        src, dst = to_dev(x, "f32"), empty_ranks(P, n, "f32")
        runs.append((fn, ref, src, dst, rc.workspace(op, P, n, torch.float32), torch.cuda.Stream()))
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(main)
    for _ in range(12):
        c = a @ b
    t1.record(main)
    ends = []
    for fn, _, src, dst, ws, s in runs:
        fn(src, dst, ws=ws, stream=s)
        e = torch.cuda.Event(enable_timing=True)
        e.record(s)
        ends.append(e)
    torch.cuda.synchronize()
    note("GEMM chain %.2f ms; ring calls ended at %s ms after its start"
         % (t0.elapsed_time(t1), ", ".join("%.2f" % t0.elapsed_time(e) for e in ends)))
    del c
    for fn, ref, src, dst, ws, s in runs:
        assert rc.last_error(ws, stream=s)[0] == 0
        np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(ref(x)), err_msg=fn.__name__)


def test_binding_refuses_a_workspace_the_kernels_cannot_use():
    """A host tensor or a strided view as the workspace is refused by the
    binding before any call; a workspace of another element type is passed
    with its size in bytes."""
    P, n = 4, 4 * 4096
    note("binding workspace checks")
    x = inputs.normal_f32(P, n, seed=1395)
    src, dst = to_dev(x, "f32"), empty_ranks(P, n, "f32")
    nb = rc.workspace_bytes(N.OP_ALL_REDUCE, P, n, torch.float32)
    with pytest.raises(ValueError):
        rc.all_reduce(src, dst, ws=torch.zeros(nb, dtype=torch.uint8))
    with pytest.raises(ValueError):
        rc.all_reduce(src, dst, ws=torch.zeros(2 * nb, dtype=torch.uint8, device="cuda")[::2])
    ws32 = torch.zeros((nb + 3) // 4, dtype=torch.int32, device="cuda")
    rc.all_reduce(src, dst, ws=ws32)
    assert rc.last_error(ws32)[0] == 0
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))


@pytest.mark.parametrize("n", [4 * 1000, 4 * (3 * 4096 + 77)])
def test_every_collective_on_buffers_4_bytes_off_alignment(n):
    """Rank buffers that start 4 bytes past a 16-byte boundary (views at
    element 1 of larger allocations) take the element-wise path: every
    collective, in the low-latency rounds (small n) and the flag rounds,
    bit for bit against the oracle."""
    P = 4
    note("unaligned bases n=%d" % n)
    x = inputs.normal_f32(P, n, seed=1460 + n % 97)

    def views(a=None):
        out = []
        for r in range(P):
            big = torch.full((n + 4,), float("nan"), dtype=torch.float32, device="cuda")
            v = big[1:n + 1]
            if a is not None:
                v.copy_(torch.from_numpy(np.ascontiguousarray(a[r])).cuda())
            out.append(v)
        return out

    src = views(x)
    assert all(t.data_ptr() % 16 == 4 for t in src)
    C = n // P
    dst = views()
    rc.ppermute(src, dst)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.ppermute(x)))
    dst = views()
    rc.all_reduce(src, dst)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_reduce(x)))
    dst = views()
    rc.reduce_scatter(src, dst)
    got, want = to_host(dst, "f32"), oracle.reduce_scatter(x)
    for r, c in rs_written_chunks(P):
        np.testing.assert_array_equal(bits(got[r, c * C:(c + 1) * C]), bits(want[r, c * C:(c + 1) * C]))
    pieces = np.stack([x[r, r * C:(r + 1) * C] for r in range(P)])
    psrc = []
    for r in range(P):
        big = torch.zeros(C + 4, dtype=torch.float32, device="cuda")
        v = big[1:C + 1]
        v.copy_(torch.from_numpy(pieces[r]).cuda())
        psrc.append(v)
    dst = views()
    rc.all_gather(dst, src=psrc)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.all_gather_pieces(pieces)))
    dst = views()
    rc.reduce_scatter_bidir(src, dst)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.reduce_scatter_bidir(x)))
    dst = views()
    rc.psum_circulating(src, dst)
    np.testing.assert_array_equal(bits(to_host(dst, "f32")), bits(oracle.psum_circulating(x)[0]))


@pytest.mark.parametrize("n", [4 * 2000, 4 * (3 * 8192 + 77)])
def test_bf16_collectives_on_buffers_2_bytes_off_alignment(n):
    """bf16 rank buffers that start 2 bytes past a 16-byte boundary: the
    fp32 carry's element-wise path in every collective that adds, in the
    low-latency and the flag rounds, bit for bit against the oracle (the
    reduce-scatters on the owners' chunks)."""
    P = 4
    note("bf16 unaligned bases n=%d" % n)
    x = inputs.normal_bf16(P, n, seed=1470 + n % 89)

    def views(a=None):
        out = []
        for r in range(P):
            big = torch.full((n + 8,), 0x7FC1, dtype=torch.int16, device="cuda")
            v = big[1:n + 1]
            if a is not None:
                v.copy_(torch.from_numpy(np.ascontiguousarray(a[r]).view(np.int16)).cuda())
            out.append(v.view(torch.bfloat16))
        return out

    src = views(x)
    assert all(t.data_ptr() % 16 == 2 for t in src)
    C = n // P
    dst = views()
    rc.all_reduce(src, dst)
    np.testing.assert_array_equal(to_host(dst, "bf16"), oracle.all_reduce_bf16(x))
    for fn, ref in ((rc.reduce_scatter, lambda v: oracle.reduce_scatter_bf16(v)[0]),
                    (rc.reduce_scatter_bidir, lambda v: oracle.reduce_scatter_bidir_bf16(v)[0])):
        dst = views()
        fn(src, dst)
        got, want = to_host(dst, "bf16"), ref(x)
        for r in range(P):
            np.testing.assert_array_equal(got[r, r * C:(r + 1) * C], want[r, r * C:(r + 1) * C],
                                          err_msg="%s rank %d" % (fn.__name__, r))
    dst = views()
    rc.psum_circulating(src, dst)
    np.testing.assert_array_equal(to_host(dst, "bf16"), oracle.psum_circulating_bf16(x))

"""GPU parity of the fused all-gather + GEMM against the CPU oracle, through
the C ABI.

The gathered A must equal the oracle's ring all-gather bit for bit.  The
products are accumulated by the matrix cores in an order the hardware fixes,
so C is compared exactly on integer-valued operands (every partial sum is an
integer below 2^24) and otherwise within |got - ref| <= K 2^-24 sum_k |a b|
against the fp64 product (recursive summation of K products; Higham,
Accuracy and Stability of Numerical Algorithms, section 3.1).
"""
import numpy as np
import pytest
import torch

import oracle
from ring_collectives_amd import _native as N
from ring_collectives_amd import collectives as rc
from ring_collectives_amd import inputs

from _gpu_helpers import note

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


@pytest.fixture(params=[128, 256])
def tile_n(request):
    N.set_tuning(gemm_tile_n=request.param)
    return request.param


def _dev_bf16(x):
    return [torch.from_numpy(np.ascontiguousarray(x[q]).view(np.int16)).cuda().view(torch.bfloat16)
            for q in range(x.shape[0])]


def _run(As, B, ws=None):
    P, Mc, K = As.shape
    Nn = B.shape[2]
    a, b = _dev_bf16(As), _dev_bf16(B)
    full = [torch.full((Mc * P, K), 0x7FC1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            for _ in range(P)]
    C = [torch.full((Mc * P, Nn), float("nan"), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws = rc.all_gather_gemm(a, b, full, C, ws=ws)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    gf = np.stack([t.view(torch.int16).cpu().numpy().view(np.uint16) for t in full])
    gc = np.stack([t.cpu().numpy() for t in C])
    return gf, gc, ws


@pytest.mark.parametrize("P,M,N,K", [(1, 256, 256, 64), (2, 512, 256, 128), (4, 1024, 512, 64),
                                     (3, 768, 384, 192), (4, 2048, 256, 128)])
def test_integer_valued_exact(P, M, N, K, tile_n):
    if tile_n == 256 and N % 256:
        pytest.skip("256-wide tiles need N % 256 == 0")
    note("ag_gemm integer P=%d M=%d N=%d K=%d tile_n=%d" % (P, M, N, K, tile_n))
    rng = np.random.default_rng(500 + P)
    As = inputs.small_int_bf16(rng, (P, M // P, K))
    B = inputs.small_int_bf16(rng, (P, K, N))
    gf, gc, _ = _run(As, B)
    want_full, want_c = oracle.all_gather_gemm(As, B)
    np.testing.assert_array_equal(gf, want_full)
    np.testing.assert_array_equal(gc.view(np.uint32), want_c.view(np.uint32))


@pytest.mark.parametrize("P,M,N,K", [(2, 512, 512, 1024), (4, 1024, 768, 512)])
def test_normal_within_bound(P, M, N, K):
    note("ag_gemm normal P=%d M=%d N=%d K=%d" % (P, M, N, K))
    As, B = inputs.gemm_operands(P, M // P, N, K, seed=510 + P)
    gf, gc, _ = _run(As, B)
    want_full, want_c = oracle.all_gather_gemm(As, B)
    np.testing.assert_array_equal(gf, want_full)
    rows = np.arange(M)
    for q in range(P):
        ref, mag = oracle.all_gather_gemm_rows_f64(As, B, q, rows)
        err = np.abs(gc[q].astype(np.float64) - ref) / mag
        assert err.max() <= K * 2.0 ** -24, (q, err.max())
    assert np.max(np.abs(gc - want_c)) <= 1e-3 * np.max(np.abs(want_c))


@pytest.mark.parametrize("P", [4, 8])
def test_full_occupancy_integer_exact(P, tile_n):
    """M = N = 4096: every CU busy, panels forwarded by many workgroups while
    others already multiply; every element of every output, three calls on
    one workspace (the panel flags must be cleared between calls)."""
    M = Nn = 4096
    K = 256
    note("ag_gemm full occupancy P=%d tile_n=%d" % (P, tile_n))
    rng = np.random.default_rng(520 + P)
    As = inputs.small_int_bf16(rng, (P, M // P, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    want_full, want_c = oracle.all_gather_gemm(As, B)
    ws = None
    for call in range(3):
        gf, gc, ws = _run(As, B, ws=ws)
        np.testing.assert_array_equal(gf, want_full, err_msg="call %d" % call)
        bad = int(np.count_nonzero(gc.view(np.uint32) != want_c.view(np.uint32)))
        assert bad == 0, "call %d: %d elements differ" % (call, bad)


def test_full_size_every_element():
    """P = 4, A 4096 x 4096 in row blocks of 1024, B_q 4096 x 4096,
    normal(0, 1/64), seed 5 (the all-gather + GEMM workload), in the default
    launch configuration: the gathered A bit for bit, and every element of
    every rank's C within K 2^-24 |A_full| |B_q| of the fp64 product (full
    host products, no sampling)."""
    P, M, Nn, K = 4, 4096, 4096, 4096
    note("ag_gemm full size generate")
    As, B = inputs.gemm_operands(P, M // P, Nn, K, seed=5)
    note("ag_gemm full size run")
    gf, gc, _ = _run(As, B)
    np.testing.assert_array_equal(gf, np.stack([As.reshape(M, K)] * P))
    assert np.all(np.isfinite(gc))
    worst = 0.0
    for q in range(P):
        note("ag_gemm full size check rank %d" % q)
        ref, mag = oracle.all_gather_gemm_f64(As, B, q)
        err = np.abs(gc[q].astype(np.float64) - ref) / mag
        worst = max(worst, float(err.max()))
    assert worst <= K * 2.0 ** -24, worst
    print("max normalised error %.3e (bound %.3e)" % (worst, K * 2.0 ** -24))


def test_errors():
    P, Mc, K, Nn = 2, 256, 64, 256
    rng = np.random.default_rng(530)
    a = _dev_bf16(inputs.small_int_bf16(rng, (P, Mc, K)))
    b = _dev_bf16(inputs.small_int_bf16(rng, (P, K, Nn)))
    full = [torch.empty((Mc * P, K), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    C = [torch.empty((Mc * P, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(N.RingError) as e:
        rc.all_gather_gemm(a, b, full, C, ws=small)
    assert e.value.code == N.RING_EWORKSPACE
    # a gathered buffer on top of a shard
    alias = [torch.empty(Mc * P * K, dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    shards = [t[:Mc * K].view(Mc, K) for t in alias]
    for s_, x in zip(shards, a):
        s_.copy_(x)
    with pytest.raises(N.RingError) as e:
        rc.all_gather_gemm(shards, b, [t.view(Mc * P, K) for t in alias], C)
    assert e.value.code == N.RING_EINVAL
    # K not a multiple of 64
    a96 = [torch.zeros((Mc, 96), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    b96 = [torch.zeros((96, Nn), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    f96 = [torch.zeros((Mc * P, 96), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    with pytest.raises(N.RingError) as e:
        rc.all_gather_gemm(a96, b96, f96, C)
    assert e.value.code == N.RING_EUNSUPPORTED


def test_watchdog_reports_timeout_and_recovers():
    """Rank 0 never flags its tiles of phase 1: its right neighbour's phase-2
    tiles wait for them, time out, and every workgroup exits; the same
    workspace then serves a normal call."""
    P, M, Nn, K = 4, 2048, 512, 128
    rng = np.random.default_rng(540)
    As = inputs.small_int_bf16(rng, (P, M // P, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    a, b = _dev_bf16(As), _dev_bf16(B)
    full = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    C = [torch.empty((M, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    note("ag_gemm watchdog drop_round=1")
    N.set_tuning(drop_round=1, timeout_s=0.05)
    ws = rc.all_gather_gemm(a, b, full, C)
    code, info = rc.last_error(ws)
    assert code == N.RING_ETIMEOUT
    N.set_tuning(drop_round=0, timeout_s=5.0)
    rc.workspace_init(ws)
    _, gc, _ = _run(As, B, ws=ws)
    _, want_c = oracle.all_gather_gemm(As, B)
    np.testing.assert_array_equal(gc.view(np.uint32), want_c.view(np.uint32))


@pytest.mark.parametrize("P,M,N,K", [(3, 768, 2048, 64), (4, 1024, 4096, 128), (2, 512, 1024, 192)])
def test_more_column_tiles_than_k_pieces(P, M, N, K, tile_n):
    """The tiles of a panel forward its K range between them, one share per
    column tile, in pieces of 8 columns: with more column tiles than pieces
    some tiles forward nothing, and the gathered buffers must still come out
    whole (pre-filled with a NaN pattern, so a hole shows), every product
    exact."""
    note("ag_gemm share split P=%d M=%d N=%d K=%d tile_n=%d" % (P, M, N, K, tile_n))
    rng = np.random.default_rng(560 + P + K)
    As = inputs.small_int_bf16(rng, (P, M // P, K))
    B = inputs.small_int_bf16(rng, (P, K, N))
    gf, gc, _ = _run(As, B)
    want_full, want_c = oracle.all_gather_gemm(As, B)
    np.testing.assert_array_equal(gf, want_full)
    np.testing.assert_array_equal(gc.view(np.uint32), want_c.view(np.uint32))


def test_more_than_64_column_tiles():
    """A panel of more than 64 column tiles: a tile of phase f >= 2 waits for
    its panel's flags 64 at a time (one lane per flag).  P = 3 so that phase
    2 waits; 256 x 128 tiles, N = 8448: 66 column tiles."""
    P, M, Nn, K = 3, 768, 8448, 64
    N.set_tuning(gemm_tile_n=128)
    note("ag_gemm 66 column tiles")
    rng = np.random.default_rng(571)
    As = inputs.small_int_bf16(rng, (P, M // P, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    gf, gc, _ = _run(As, B)
    want_full, want_c = oracle.all_gather_gemm(As, B)
    np.testing.assert_array_equal(gf, want_full)
    np.testing.assert_array_equal(gc.view(np.uint32), want_c.view(np.uint32))


def _random_shapes(seed, count):
    """Seeded shapes the kernel accepts: P of 2..8 (5, 6 and 7 included),
    row blocks of one or two 256-row tiles per rank, N a multiple of 128,
    K a multiple of 64."""
    rng = np.random.default_rng(seed)
    out = []
    for P in (5, 6, 7, 3, 8, 2)[:count]:
        out.append((P, 256 * P * int(rng.integers(1, 3)), 128 * int(rng.integers(1, 6)), 64 * int(rng.integers(1, 6))))
    return out


@pytest.mark.parametrize("P,M,N,K", _random_shapes(1420, 6))
def test_random_shapes_integer_exact(P, M, N, K):
    """Odd rank counts and sizes with the automatic tile width: the gathered
    rows and every product bit, against the oracle."""
    note("ag_gemm random P=%d M=%d N=%d K=%d" % (P, M, N, K))
    rng = np.random.default_rng(1430 + P)
    As = inputs.small_int_bf16(rng, (P, M // P, K))
    B = inputs.small_int_bf16(rng, (P, K, N))
    gf, gc, _ = _run(As, B)
    want_full, want_c = oracle.all_gather_gemm(As, B)
    np.testing.assert_array_equal(gf, want_full)
    np.testing.assert_array_equal(gc.view(np.uint32), want_c.view(np.uint32))


@pytest.mark.parametrize("P,M,N,K", [(16, 4096, 256, 128), (32, 8192, 128, 64), (64, 16384, 128, 64)])
def test_many_ranks_integer_exact(P, M, N, K):
    """16, 32 and 64 ranks (the library's maximum): the gathered A and every
    bit of C against the oracle."""
    note("ag_gemm many ranks P=%d M=%d N=%d K=%d" % (P, M, N, K))
    rng = np.random.default_rng(1430 + P)
    As = inputs.small_int_bf16(rng, (P, M // P, K))
    B = inputs.small_int_bf16(rng, (P, K, N))
    gf, gc, _ = _run(As, B)
    want_full, want_c = oracle.all_gather_gemm(As, B)
    np.testing.assert_array_equal(gf, want_full)
    np.testing.assert_array_equal(gc.view(np.uint32), want_c.view(np.uint32))


def test_repeated_calls_with_new_inputs_on_the_same_buffers(tile_n):
    """Three calls, each with new shards and weights, into the same gathered
    buffers, outputs and workspace: the tiles of phases 2 and up read the
    gathered rows with ordinary (cached) loads, so every call must see the
    rows its own launch forwarded, not what an earlier call left there.
    K = 192 splits the forwarding shares inside 128-byte lines (48 or 96
    elements per column tile), so lines are written piecewise by several
    tiles before they are read."""
    P, M, Nn, K = 4, 1024, 512, 192
    note("ag_gemm repeated calls with new inputs tile_n=%d" % tile_n)
    full = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    C = [torch.empty((M, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws = None
    for call in range(3):
        rng = np.random.default_rng(1450 + call)
        As = inputs.small_int_bf16(rng, (P, M // P, K))
        B = inputs.small_int_bf16(rng, (P, K, Nn))
        ws = rc.all_gather_gemm(_dev_bf16(As), _dev_bf16(B), full, C, ws=ws)
        torch.cuda.synchronize()
        assert rc.last_error(ws)[0] == 0
        want_full, want_c = oracle.all_gather_gemm(As, B)
        gf = np.stack([t.view(torch.int16).cpu().numpy().view(np.uint16) for t in full])
        gc = np.stack([t.cpu().numpy() for t in C])
        np.testing.assert_array_equal(gf, want_full, err_msg="call %d" % call)
        np.testing.assert_array_equal(gc.view(np.uint32), want_c.view(np.uint32), err_msg="call %d" % call)

"""GPU parity of the fused GEMM + reduce-scatter against the CPU oracle.

The per-rank products are accumulated by the matrix cores in an order the
hardware fixes, so general inputs are compared within a bound: componentwise,
|got - ref| <= (K + P) 2^-24 * sum_q sum_k |A_q[i,k] B_q[k,j]| (recursive
summation of K products, then P - 1 ring additions; Higham, Accuracy and
Stability of Numerical Algorithms, section 3.1), with ref the fp64 value.
Two input families are exact in any order and compared bit for bit:
integer-valued operands, and a diagonal A (each output is one exact product),
which leaves only the ring's fp32 additions -- so the reduce-scatter order is
checked bit for bit against the oracle's.
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


@pytest.fixture(params=[64, 128, 256])
def tile_n(request):
    """Every output tile width: 256 x 64 (one workgroup per compute unit),
    256 x 128 (two) and 256 x 256 (one)."""
    old = N.set_tuning(gemm_tile_n=request.param)
    yield request.param
    N.set_tuning(gemm_tile_n=old["gemm_tile_n"])


def _dev_bf16(x):
    return [torch.from_numpy(np.ascontiguousarray(x[q]).view(np.int16)).cuda().view(torch.bfloat16)
            for q in range(x.shape[0])]


def _run(A, B, ws=None):
    P, M, K = A.shape
    Nn = B.shape[2]
    a, b = _dev_bf16(A), _dev_bf16(B)
    out = [torch.full((M // P, Nn), float("nan"), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws = rc.gemm_reduce_scatter(a, b, out, ws=ws)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    return np.stack([o.cpu().numpy() for o in out]), ws


@pytest.mark.parametrize("P,M,N,K", [(1, 256, 256, 64), (2, 512, 256, 128), (4, 1024, 512, 64),
                                     (4, 2048, 256, 192), (3, 768, 768, 64)])
def test_integer_valued_exact(P, M, N, K, tile_n):
    note("gemm_rs integer P=%d M=%d N=%d K=%d tile_n=%d" % (P, M, N, K, tile_n))
    rng = np.random.default_rng(200 + P)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, N))
    got, _ = _run(A, B)
    Ai = oracle.bf16_to_f32(A).astype(np.int64)
    Bi = oracle.bf16_to_f32(B).astype(np.int64)
    total = sum(Ai[q] @ Bi[q] for q in range(P))
    rows = M // P
    for r in range(P):
        np.testing.assert_array_equal(got[r].astype(np.int64), total[r * rows:(r + 1) * rows],
                                      err_msg="rank %d" % r)


@pytest.mark.parametrize("P", [2, 3, 4])
def test_diagonal_a_ring_order_bit_exact(P, tile_n):
    """A_q = diag(a_q): every product is exact in fp32, so only the ring's
    fp32 additions round, and they must match the oracle bit for bit."""
    note("gemm_rs diagonal P=%d tile_n=%d" % (P, tile_n))
    M = 256 * P * 2
    rng = np.random.default_rng(300 + P)
    a = inputs.bf16_bits(rng.standard_normal((P, M)).astype(np.float32))
    A = np.zeros((P, M, M), dtype=np.uint16)
    for q in range(P):
        A[q][np.arange(M), np.arange(M)] = a[q]
    # wide dynamic range so the association order shows in the bits
    Bf = rng.standard_normal((P, M, 512)).astype(np.float32) * np.exp2(rng.integers(-12, 12, size=(P, M, 512))).astype(np.float32)
    B = inputs.bf16_bits(Bf)
    got, _ = _run(A, B)
    want = oracle.gemm_reduce_scatter(A, B)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("P,M,N,K", [(1, 256, 512, 512), (2, 512, 512, 1024), (4, 1024, 768, 512)])
def test_normal_within_bound(P, M, N, K):
    note("gemm_rs normal P=%d M=%d N=%d K=%d" % (P, M, N, K))
    A, B = inputs.gemm_operands(P, M, N, K, seed=400 + P)
    got, _ = _run(A, B)
    rows = M // P
    for r in range(P):
        ref, mag = oracle.gemm_reduce_scatter_rows_f64(A, B, r, np.arange(rows))
        err = np.abs(got[r].astype(np.float64) - ref) / mag
        assert err.max() <= (K + P) * 2.0 ** -24, (r, err.max())
    # and against the oracle's fp32 pipeline (fp64 products rounded, ring adds)
    want = oracle.gemm_reduce_scatter(A, B)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - want)) <= 1e-3 * np.max(np.abs(want))


@pytest.mark.parametrize("P", [4, 8])
def test_full_occupancy_integer_exact(P, tile_n):
    """M = N = 4096: enough tiles that every compute unit holds as many
    workgroups as it can, with rings of neighbouring ranks running in
    different phases at once.  Integer-valued operands make every output
    exact, so all elements are compared bit for bit, over repeated calls on
    one workspace."""
    M = Nn = 4096
    K = 256
    note("gemm_rs full occupancy P=%d tile_n=%d" % (P, tile_n))
    rng = np.random.default_rng(600 + P)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    want = oracle.gemm_reduce_scatter(A, B)
    a, b = _dev_bf16(A), _dev_bf16(B)
    ws = None
    for call in range(3):
        out = [torch.full((M // P, Nn), float("nan"), dtype=torch.float32, device="cuda") for _ in range(P)]
        ws = rc.gemm_reduce_scatter(a, b, out, ws=ws)
        torch.cuda.synchronize()
        assert rc.last_error(ws)[0] == 0
        got = np.stack([o.cpu().numpy() for o in out])
        bad = int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
        assert bad == 0, "call %d: %d elements differ" % (call, bad)


@pytest.fixture(scope="module")
def full_size():
    """P = 4, A_q and B_q bf16 4096 x 4096, normal(0, 1/64), seed 4 (the
    workload of the collective-matmul GEMM + reduce-scatter), on the device."""
    P, M, Nn, K = 4, 4096, 4096, 4096
    note("gemm_rs full size generate")
    A, B = inputs.gemm_operands(P, M, Nn, K)
    return A, B, _dev_bf16(A), _dev_bf16(B)


def _fused(a, b, P, M, Nn):
    out = [torch.full((M // P, Nn), float("nan"), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws = rc.gemm_reduce_scatter(a, b, out)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    return np.stack([o.cpu().numpy() for o in out])


def test_full_size_every_element(full_size):
    """Every element of every rank's output, in the default launch
    configuration, within (K + P) 2^-24 sum_q |A_q||B_q| of the fp64 sum
    (full host products, no sampling)."""
    A, B, a, b = full_size
    P, M, K = A.shape
    Nn = B.shape[2]
    note("gemm_rs full size run")
    got = _fused(a, b, P, M, Nn)
    assert np.all(np.isfinite(got))
    worst = 0.0
    for r in range(P):
        note("gemm_rs full size check rank %d" % r)
        ref, mag = oracle.gemm_reduce_scatter_f64(A, B, r)
        err = np.abs(got[r].astype(np.float64) - ref) / mag
        worst = max(worst, float(err.max()))
    assert worst <= (K + P) * 2.0 ** -24, worst
    print("max normalised error %.3e (bound %.3e)" % (worst, (K + P) * 2.0 ** -24))


@pytest.mark.parametrize("bn", [256, 128])
def test_full_size_ring_part_bit_exact_on_own_products(full_size, bn):
    """The reduce-scatter part on the kernel's own products, bit for bit: each
    C_q comes from the same kernel's P = 1 path (same tile width, same K
    order, no ring), the oracle's fp32 ring reduce-scatter runs over those
    products, and the fused output must equal it on every element -- the
    ring's association order ((C_{c+1} + C_{c+2}) + ...) + C_c at full size
    on the workload's data."""
    A, B, a, b = full_size
    P, M, K = A.shape
    Nn = B.shape[2]
    old = N.set_tuning(gemm_tile_n=bn)
    try:
        note("gemm_rs own products P=1 x %d, tile_n=%d" % (P, bn))
        C = [torch.full((M, Nn), float("nan"), dtype=torch.float32, device="cuda") for _ in range(P)]
        ws1 = None
        for q in range(P):
            ws1 = rc.gemm_reduce_scatter([a[q]], [b[q]], [C[q]], ws=ws1)
        torch.cuda.synchronize()
        assert rc.last_error(ws1)[0] == 0
        products = np.stack([c.cpu().numpy() for c in C])
        del C
        note("gemm_rs fused, tile_n=%d" % bn)
        got = _fused(a, b, P, M, Nn)
    finally:
        N.set_tuning(gemm_tile_n=old["gemm_tile_n"])
    st = oracle.reduce_scatter(products.reshape(P, M * Nn))
    rows = M // P
    for r in range(P):
        want = st[r].reshape(M, Nn)[r * rows:(r + 1) * rows]
        bad = int(np.count_nonzero(got[r].view(np.uint32) != want.view(np.uint32)))
        assert bad == 0, "rank %d: %d elements differ" % (r, bad)


def test_narrow_n_uses_128_wide_tiles():
    """N = 384 is a multiple of 128 but not of 256: the automatic choice
    takes 256 x 128 tiles and the result is exact; forcing 256-wide tiles is
    rejected before any launch."""
    P, M, Nn, K = 2, 512, 384, 128
    note("gemm_rs N=384")
    rng = np.random.default_rng(8)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    assert N.get_tuning()["gemm_tile_n"] == 0
    got, _ = _run(A, B)
    want = oracle.gemm_reduce_scatter(A, B)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    old = N.set_tuning(gemm_tile_n=256)
    try:
        a, b = _dev_bf16(A), _dev_bf16(B)
        out = [torch.empty((M // P, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
        with pytest.raises(N.RingError) as e:
            rc.gemm_reduce_scatter(a, b, out)
        assert e.value.code == N.RING_EUNSUPPORTED
    finally:
        N.set_tuning(gemm_tile_n=old["gemm_tile_n"])


def test_repeated_calls_and_errors():
    P, M, Nn, K = 4, 1024, 256, 128
    rng = np.random.default_rng(7)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    got1, ws = _run(A, B)
    got2, _ = _run(A, B, ws=ws)
    np.testing.assert_array_equal(got1, got2)
    a, b = _dev_bf16(A), _dev_bf16(B)
    out = [torch.empty((M // P, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    # K = 96 is not a multiple of 64: rejected before any launch
    a96 = [x[:, :96].contiguous() for x in a]
    b96 = [x[:96].contiguous() for x in b]
    with pytest.raises(N.RingError) as e:
        rc.gemm_reduce_scatter(a96, b96, out)
    assert e.value.code == N.RING_EUNSUPPORTED
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(N.RingError) as e:
        rc.gemm_reduce_scatter(a, b, out, ws=small)
    assert e.value.code == N.RING_EWORKSPACE


def _random_shapes(seed, count):
    """Seeded shapes the kernel accepts: P of 2..8 (5, 6 and 7 included),
    row blocks of one or two 256-row tiles per rank, N a multiple of 128,
    K a multiple of 64."""
    rng = np.random.default_rng(seed)
    out = []
    for P in (5, 6, 7, 3, 8, 2)[:count]:
        out.append((P, 256 * P * int(rng.integers(1, 3)), 128 * int(rng.integers(1, 6)), 64 * int(rng.integers(1, 6))))
    return out


@pytest.mark.parametrize("P,M,N,K", _random_shapes(1400, 6))
def test_random_shapes_integer_exact(P, M, N, K):
    """Odd rank counts and sizes with the automatic tile width: every bit,
    against the oracle."""
    note("gemm_rs random P=%d M=%d N=%d K=%d" % (P, M, N, K))
    rng = np.random.default_rng(1410 + P)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, N))
    got, _ = _run(A, B)
    want = oracle.gemm_reduce_scatter(A, B)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_beside_vendor_gemms_on_another_stream():
    """GEMM + RS on a side stream while a chain of vendor GEMMs holds the
    GPU: its workgroups that start first wait for the rest, which start as
    the other kernel's workgroups finish, so the call is only delayed (well
    within the watchdog); integer-valued operands, every element exact."""
    P, M, Nn, K = 4, 2048, 1024, 512
    note("gemm_rs beside vendor GEMMs on another stream")
    rng = np.random.default_rng(1390)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, Nn))
    a, b = _dev_bf16(A), _dev_bf16(B)
    out = [torch.full((M // P, Nn), float("nan"), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws = rc.workspace(N.OP_GEMM_REDUCE_SCATTER, P, M * Nn, torch.float32)
    x = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(8):
        z = x @ y
    rc.gemm_reduce_scatter(a, b, out, ws=ws, stream=side)
    torch.cuda.synchronize()
    del z
    assert rc.last_error(ws, stream=side)[0] == 0
    got = np.stack([o.cpu().numpy() for o in out])
    np.testing.assert_array_equal(got.view(np.uint32), oracle.gemm_reduce_scatter(A, B).view(np.uint32))


@pytest.mark.parametrize("P,M,N,K", [(16, 4096, 256, 128), (32, 8192, 128, 64), (64, 16384, 128, 64)])
def test_many_ranks_integer_exact(P, M, N, K):
    """16, 32 and 64 ranks (the library's maximum), one 256-row tile per rank
    and chunk, the automatic tile width: every bit against the oracle."""
    note("gemm_rs many ranks P=%d M=%d N=%d K=%d" % (P, M, N, K))
    rng = np.random.default_rng(1420 + P)
    A = inputs.small_int_bf16(rng, (P, M, K))
    B = inputs.small_int_bf16(rng, (P, K, N))
    got, _ = _run(A, B)
    np.testing.assert_array_equal(got.view(np.uint32), oracle.gemm_reduce_scatter(A, B).view(np.uint32))

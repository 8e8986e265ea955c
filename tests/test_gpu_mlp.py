"""GPU parity of the tensor-parallel MLP layer against the CPU oracle
("TPU 与分布式通信原语", collective matmul: out_shard = ReduceScatter(
gelu(AllGather(x_shard) @ W1_i) @ W2_i)), through the C ABI.

The gathered input must equal the oracle's ring all-gather bit for bit.  The
products are accumulated by the matrix cores in an order the hardware fixes
and gelu is evaluated in fp32, so:
  * on integer-valued operands whose every partial sum is exact in fp32, h
    and the output are compared bit for bit;
  * on the workload's inputs (x and W1 on fixed-point grids, which makes the
    first product exact) every h must lie in the oracle's interval -- one
    value except where gelu's fp32 evaluation error reaches a bf16 rounding
    boundary -- and every output in [bf16(s - t), bf16(s + t)] with s the
    fp64 sum and t the fp32 error bound of the second product and the ring
    sum (oracle.tp_mlp_bounds).
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


@pytest.fixture(params=[64, 128, 256])
def tile_n(request):
    N.set_tuning(gemm_tile_n=request.param)
    return request.param


def _dev(a):
    return [torch.from_numpy(np.ascontiguousarray(a[q]).view(np.int16)).cuda().view(torch.bfloat16)
            for q in range(a.shape[0])]


def _host(ts):
    return np.stack([t.view(torch.int16).cpu().numpy().view(np.uint16) for t in ts])


def _nan_bf16(shape):
    return torch.full(shape, 0x7FC1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _run(x, w1, w2, ws=None, out=None):
    P, Mq, D = x.shape
    Fr = w1.shape[2]
    M = Mq * P
    xs, W1, W2 = _dev(x), _dev(w1), _dev(w2)
    full = [_nan_bf16((M, D)) for _ in range(P)]
    h = [_nan_bf16((M, Fr)) for _ in range(P)]
    out = [_nan_bf16((Mq, D)) for _ in range(P)] if out is None else out
    ws = rc.tp_mlp_layer(xs, W1, W2, full, h, out, ws=ws)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    return _host(full), _host(h), _host(out), ws


def _int_operands(P, M, D, F, seed):
    """x rows with three ones, W1 in {0, 1}: x @ W1 in {0..3}, so h is one of
    bf16(gelu(0..3)) = 0, 215/256, 250/128, 3; W2 in {-1, 0, 1}: every
    partial sum of the second product and of the ring is a multiple of 2^-8
    below 2^16 in magnitude, exact in fp32."""
    rng = np.random.default_rng(seed)
    Mq, Fr = M // P, F // P
    x = np.zeros((P, Mq, D), dtype=np.float32)
    for q in range(P):
        for i in range(Mq):
            x[q, i, rng.choice(D, size=3, replace=False)] = 1.0
    w1 = rng.integers(0, 1, size=(P, D, Fr), endpoint=True).astype(np.float32)
    w2 = rng.integers(-1, 1, size=(P, Fr, D), endpoint=True).astype(np.float32)
    assert F * 3 * 256 < 2 ** 24
    return inputs.bf16_bits(x), inputs.bf16_bits(w1), inputs.bf16_bits(w2)


@pytest.mark.parametrize("P,M,D,F", [(1, 256, 128, 128), (2, 512, 256, 256), (4, 1024, 128, 512),
                                     (3, 768, 384, 384), (4, 2048, 256, 1024)])
def test_integer_valued_exact(P, M, D, F, tile_n):
    if tile_n == 256 and (D % 256 or (F // P) % 256):
        pytest.skip("256-wide tiles need both products' N % 256 == 0")
    note("tp_mlp integer P=%d M=%d D=%d F=%d tile_n=%d" % (P, M, D, F, tile_n))
    x, w1, w2 = _int_operands(P, M, D, F, seed=600 + P)
    gf, gh, go, _ = _run(x, w1, w2)
    full, h, out = oracle.tp_mlp_layer(x, w1, w2)
    np.testing.assert_array_equal(gf, full)
    np.testing.assert_array_equal(gh, h)
    np.testing.assert_array_equal(go, out)


def _check_bounds(x, w1, w2, gh, go, ranks_rows):
    P, Mq, _ = x.shape
    ambiguous = 0
    total = 0
    for r, rows in ranks_rows:
        _, lo, hi, s, t = oracle.tp_mlp_bounds(x, w1, w2, r, rows)
        for q in range(P):
            hv = oracle.bf16_to_f32(gh[q][r * Mq + rows]).astype(np.float64)
            bad = ~((lo[q] <= hv) & (hv <= hi[q]))
            assert not bad.any(), "h of rank %d, rows of block %d: %d outside" % (q, r, int(bad.sum()))
            ambiguous += int(np.count_nonzero(lo[q] != hi[q]))
            total += lo[q].size
        ov = oracle.bf16_to_f32(go[r][rows]).astype(np.float64)
        lo_o, hi_o = oracle.bf16_nearest(s - t), oracle.bf16_nearest(s + t)
        bad = ~((lo_o <= ov) & (ov <= hi_o))
        assert not bad.any(), "out of rank %d: %d outside" % (r, int(bad.sum()))
    # the check is tight: h has one admissible value almost everywhere
    assert ambiguous <= 0.01 * total, (ambiguous, total)


@pytest.mark.parametrize("P,M,D,F", [(2, 512, 256, 512), (4, 1024, 512, 1024), (3, 768, 128, 768)])
def test_grid_inputs_within_bounds(P, M, D, F, tile_n):
    if tile_n == 256 and (D % 256 or (F // P) % 256):
        pytest.skip("256-wide tiles need both products' N % 256 == 0")
    note("tp_mlp grid P=%d M=%d D=%d F=%d tile_n=%d" % (P, M, D, F, tile_n))
    x, w1, w2 = inputs.mlp_operands(P, M, D, F, seed=610 + P)
    gf, gh, go, _ = _run(x, w1, w2)
    full, h, out = oracle.tp_mlp_layer(x, w1, w2)
    np.testing.assert_array_equal(gf, full)
    Mq = M // P
    _check_bounds(x, w1, w2, gh, go, [(r, np.arange(Mq)) for r in range(P)])
    # and mostly the oracle's own bits
    assert np.mean(gh == h) > 0.99
    assert np.mean(go == out) > 0.9


@pytest.mark.parametrize("bn", [0, 128])
@pytest.mark.parametrize("P,M,D,F", [(4, 256, 1024, 16384), (2, 256, 256, 512), (4, 512, 256, 1024),
                                     (8, 256, 128, 1024)])
def test_small_token_counts_integer_exact(P, M, D, F, bn):
    """Fewer than 256 tokens per rank run the unfused steps (the chapter's
    own x [256, 1024], W1 [1024, 16384] at P = 4 among them): every bit,
    with the automatic tile widths (64 for these few tiles) and with 128."""
    N.set_tuning(gemm_tile_n=bn)
    note("tp_mlp unfused integer P=%d M=%d D=%d F=%d bn=%d" % (P, M, D, F, bn))
    x, w1, w2 = _int_operands(P, M, D, F, seed=660 + P)
    gf, gh, go, _ = _run(x, w1, w2)
    full, h, out = oracle.tp_mlp_layer(x, w1, w2)
    np.testing.assert_array_equal(gf, full)
    np.testing.assert_array_equal(gh, h)
    np.testing.assert_array_equal(go, out)


def test_page_shape_within_bounds_and_repeated():
    """x [256, 1024] in row blocks of 64, W1 [1024, 16384], W2 [16384, 1024],
    P = 4, the workload's distributions: every token within the oracle's
    intervals; a second call on the same workspace gives the same bits."""
    P, M, D, F = 4, 256, 1024, 16384
    note("tp_mlp page shape")
    x, w1, w2 = inputs.mlp_operands(P, M, D, F, seed=670)
    gf, gh, go, ws = _run(x, w1, w2)
    np.testing.assert_array_equal(gf, np.stack([x.reshape(M, D)] * P))
    _check_bounds(x, w1, w2, gh, go, [(r, np.arange(M // P)) for r in range(P)])
    _, gh2, go2, _ = _run(x, w1, w2, ws=ws)
    np.testing.assert_array_equal(gh2, gh)
    np.testing.assert_array_equal(go2, go)


def test_gelu_epilogue_over_its_range():
    """One rank, x rows that are unit vectors: row i of x @ W1 is row i % D of
    W1, which holds every bf16 value of a dense sweep of [-11, 11] (gelu's
    result is subnormal in fp32 below about -10.3 and zero below -10.9):
    gelu's fp32 evaluation and both bf16 roundings against the oracle,
    value by value."""
    sweep = np.concatenate([np.linspace(-11, 11, 6001), np.geomspace(1e-8, 1, 800), -np.geomspace(1e-8, 1, 800)])
    vals = np.unique(oracle.bf16_to_f32(inputs.bf16_bits(sweep.astype(np.float32))))
    F = -(-len(vals) // 128) * 128
    grid = np.concatenate([vals, vals[:F - len(vals)]]).astype(np.float32)
    P, M, D = 1, 256, 128
    rng = np.random.default_rng(620)
    w1 = np.zeros((1, D, F), dtype=np.float32)
    for k in range(D):
        w1[0, k] = rng.permutation(grid)
    x = np.zeros((1, M, D), dtype=np.float32)
    x[0, np.arange(M), np.arange(M) % D] = 1.0
    w2 = np.zeros((1, F, D), dtype=np.float32)
    xb, w1b, w2b = inputs.bf16_bits(x), inputs.bf16_bits(w1), inputs.bf16_bits(w2)
    note("tp_mlp gelu range, %d values" % len(vals))
    _, gh, _, _ = _run(xb, w1b, w2b)
    h_ref, lo, hi, _, _ = oracle.tp_mlp_bounds(xb, w1b, w2b, 0, np.arange(M))
    hv = oracle.bf16_to_f32(gh[0]).astype(np.float64)
    bad = ~((lo[0] <= hv) & (hv <= hi[0]))
    assert not bad.any(), list(zip(oracle.bf16_to_f32(w1b[0][np.arange(M) % D][bad])[:5], hv[bad][:5],
                                    lo[0][bad][:5], hi[0][bad][:5]))
    assert np.count_nonzero(lo != hi) <= 0.01 * lo.size
    assert np.mean(gh == h_ref) > 0.99


def _every_finite_bf16_layer(P, tile, D=256, F=256):
    """A layer whose first product's outputs are every finite bf16 value:
    rank q's W1 holds the values (each rank the same), x's rows are unit
    vectors, so h[q][i] = gelu(W1 row i % D).  Returns (w1 bits, h)."""
    u = np.arange(65536, dtype=np.uint32)
    vals = u[((u >> 7) & 0xFF) != 255].astype(np.uint16)
    vals = np.concatenate([vals, vals[:D * F - len(vals)]])
    M = 256
    w1b = np.stack([vals.reshape(D, F)] * P)
    x = np.zeros((P, M // P, D), dtype=np.float32)
    rows = np.arange(M)
    x.reshape(M, D)[rows, rows % D] = 1.0
    w2b = np.zeros((P, F, D), dtype=np.uint16)
    N.set_tuning(gemm_tile_n=tile)
    _, gh, _, _ = _run(inputs.bf16_bits(x), w1b, w2b)
    return w1b, gh


def test_gelu_epilogue_on_every_bf16():
    """Every finite bf16 input of the activation (65,280 values, subnormals
    included) through the epilogues of both GEMM kernels and three tile
    widths: all-gather + GEMM with 256 x 128 and 256 x 256 tiles (P = 1,
    fused) and the batched products of the unfused layer (P = 2, 256 x 64
    tiles).  The bits must agree, and lie within the oracle's intervals."""
    note("tp_mlp gelu: every finite bf16")
    w1b, h_128 = _every_finite_bf16_layer(1, 128)
    _, h_256 = _every_finite_bf16_layer(1, 256)
    _, h_unfused = _every_finite_bf16_layer(2, 0)
    np.testing.assert_array_equal(h_256, h_128)
    for q in range(2):
        np.testing.assert_array_equal(h_unfused[q], h_128[0])
    x = np.zeros((1, 256, 256), dtype=np.float32)
    x[0, np.arange(256), np.arange(256)] = 1.0
    _, lo, hi, _, _ = oracle.tp_mlp_bounds(inputs.bf16_bits(x), w1b[:1], np.zeros((1, 256, 256), np.uint16), 0,
                                           np.arange(256))
    hv = oracle.bf16_to_f32(h_128[0]).astype(np.float64)
    bad = ~((lo[0] <= hv) & (hv <= hi[0]))
    assert not bad.any(), int(bad.sum())


def test_full_size_sampled_rows():
    """P = 4, x [8192, 1024] in row blocks of 2048, W1 [1024, 16384],
    W2 [16384, 1024] in the default launch configuration: the gathered input
    everywhere, sampled tokens of h and of every rank's output."""
    P, M, D, F = 4, 8192, 1024, 16384
    note("tp_mlp full size generate")
    x, w1, w2 = inputs.mlp_operands(P, M, D, F, seed=inputs.SEED_MLP)
    note("tp_mlp full size run")
    gf, gh, go, _ = _run(x, w1, w2)
    for q in range(P):
        np.testing.assert_array_equal(gf[q], x.reshape(M, D))
    Mq = M // P
    rows = np.unique(np.concatenate([[0, 255, 256, Mq - 1], np.random.default_rng(7).integers(0, Mq, 6)]))
    note("tp_mlp full size check")
    _check_bounds(x, w1, w2, gh, go, [(r, rows) for r in range(P)])


def test_layers_in_place_match_out_of_place():
    """Two layers with each output written over its input shard give the
    bits of two layers with separate buffers, on one workspace."""
    P, M, D, F = 4, 1024, 256, 1024
    x, w1, w2 = inputs.mlp_operands(P, M, D, F, seed=630)
    _, v1, u1 = inputs.mlp_operands(P, M, D, F, seed=631)
    Mq, Fr = M // P, F // P
    bf = torch.bfloat16
    full = [torch.empty((M, D), dtype=bf, device="cuda") for _ in range(P)]
    h = [torch.empty((M, Fr), dtype=bf, device="cuda") for _ in range(P)]
    a, b = _dev(x), [torch.empty((Mq, D), dtype=bf, device="cuda") for _ in range(P)]
    c = [torch.empty((Mq, D), dtype=bf, device="cuda") for _ in range(P)]
    ws = rc.tp_mlp_workspace(P, M, D, F)
    note("tp_mlp two layers out of place")
    rc.tp_mlp_layer(a, _dev(w1), _dev(w2), full, h, b, ws=ws)
    rc.tp_mlp_layer(b, _dev(v1), _dev(u1), full, h, c, ws=ws)
    want = _host(c)
    note("tp_mlp two layers in place")
    y = _dev(x)
    rc.tp_mlp_layer(y, _dev(w1), _dev(w2), full, h, y, ws=ws)
    rc.tp_mlp_layer(y, _dev(v1), _dev(u1), full, h, y, ws=ws)
    torch.cuda.synchronize()
    assert rc.last_error(ws)[0] == 0
    np.testing.assert_array_equal(_host(y), want)
    # the first layer alone against the oracle
    _, _, out1 = oracle.tp_mlp_layer(x, w1, w2)
    assert np.mean(_host(b) == out1) > 0.9


def test_errors():
    P, M, D, F = 2, 512, 128, 256
    x, w1, w2 = inputs.mlp_operands(P, M, D, F, seed=640)
    xs, W1, W2 = _dev(x), _dev(w1), _dev(w2)
    bf = torch.bfloat16
    full = [torch.empty((M, D), dtype=bf, device="cuda") for _ in range(P)]
    h = [torch.empty((M, F // P), dtype=bf, device="cuda") for _ in range(P)]
    out = [torch.empty((M // P, D), dtype=bf, device="cuda") for _ in range(P)]
    small = torch.zeros(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(N.RingError) as e:
        rc.tp_mlp_layer(xs, W1, W2, full, h, out, ws=small)
    assert e.value.code == N.RING_EWORKSPACE
    # h on top of the gathered input (both M x 128 here)
    alias = [full[0].view(-1)[:M * (F // P)].view(M, F // P), h[1]]
    with pytest.raises(N.RingError) as e:
        rc.tp_mlp_layer(xs, W1, W2, full, alias, out)
    assert e.value.code == N.RING_EINVAL
    # out on top of h
    with pytest.raises(N.RingError) as e:
        rc.tp_mlp_layer(xs, W1, W2, full, h, [h[0].view(-1)[:(M // P) * D].view(M // P, D), out[1]])
    assert e.value.code == N.RING_EINVAL
    assert int(N.lib().tp_mlp_workspace_bytes(P, M, 96, F)) == 0
    assert int(N.lib().tp_mlp_workspace_bytes(P, 300, D, F)) == 0


def test_watchdog_reports_timeout_and_recovers():
    """Rank 0 never flags its tiles of the all-gather's phase 1: the layer
    ends in RING_ETIMEOUT; the same workspace, cleared, then serves a normal
    call."""
    P, M, D, F = 4, 1024, 256, 1024
    x, w1, w2 = _int_operands(P, M, D, F, seed=650)
    note("tp_mlp watchdog drop_round=1")
    N.set_tuning(drop_round=1, timeout_s=0.05)
    xs, W1, W2 = _dev(x), _dev(w1), _dev(w2)
    bf = torch.bfloat16
    full = [torch.empty((M, D), dtype=bf, device="cuda") for _ in range(P)]
    h = [torch.empty((M, F // P), dtype=bf, device="cuda") for _ in range(P)]
    out = [torch.empty((M // P, D), dtype=bf, device="cuda") for _ in range(P)]
    ws = rc.tp_mlp_layer(xs, W1, W2, full, h, out)
    code, _ = rc.last_error(ws)
    assert code == N.RING_ETIMEOUT
    N.set_tuning(drop_round=0, timeout_s=5.0)
    rc.workspace_init(ws)
    _, gh, go, _ = _run(x, w1, w2, ws=ws)
    _, h_ref, out_ref = oracle.tp_mlp_layer(x, w1, w2)
    np.testing.assert_array_equal(gh, h_ref)
    np.testing.assert_array_equal(go, out_ref)


def _random_mlp_shapes(seed):
    """Seeded layer shapes with rank counts 3, 5, 6 and 7: fused ones (256 P
    or 512 P tokens) and, for P = 6, the unfused path (768 tokens: 128 per
    rank; with an odd P the token count, a multiple of 256 and of P, is
    always a multiple of 256 P).  D a multiple of 128, F of 128 P."""
    rng = np.random.default_rng(seed)
    out = []
    for P, M in ((3, 768 * int(rng.integers(1, 3))), (5, 1280), (6, 768), (6, 1536), (7, 1792)):
        out.append((P, M, 128 * int(rng.integers(1, 3)), 128 * P * int(rng.integers(1, 4))))
    return out


@pytest.mark.parametrize("P,M,D,F", _random_mlp_shapes(1440))
def test_random_shapes_integer_exact(P, M, D, F):
    """Rank counts 3, 5, 6 and 7 on both paths with the automatic tile
    widths: the gathered activations, h and the output, every bit."""
    note("tp_mlp random P=%d M=%d D=%d F=%d" % (P, M, D, F))
    x, w1, w2 = _int_operands(P, M, D, F, seed=1450 + P)
    gf, gh, go, _ = _run(x, w1, w2)
    full, h, out = oracle.tp_mlp_layer(x, w1, w2)
    np.testing.assert_array_equal(gf, full)
    np.testing.assert_array_equal(gh, h)
    np.testing.assert_array_equal(go, out)


@pytest.mark.parametrize("P,M,D,F", [(4, 256, 1024, 16384), (4, 1024, 1024, 16384)])
def test_plain_normal_operands(P, M, D, F):
    """Plain normal bf16 operands, no grid (x normal(0, 1), W1 normal(0,
    1/D), W2 normal(0, 1/F)), at the chapter's shape (x [256, 1024] over four
    ranks: the unfused path) and at 1024 tokens (the fused kernels), in the
    default launch configuration.  The first product is now inexact in fp32,
    so the oracle's intervals take its recursive-summation bound.
      * every element of h and of the output lies in the oracle's intervals
        (rigorous: fp32 in any order, gelu within its fp32 allowance);
      * those worst-case intervals are wide for a 1024- and a 4096-term fp32
        sum, so the layer is also held to the oracle's own bits.  The bf16
        rounding of an fp32 product differs from the oracle's (the exact
        product rounded once) only where the product lies within its fp32
        rounding error, about 2^-19 relative for these sums, of a bf16
        rounding boundary (spaced 2^-8): about 0.05% of h; the output's sums
        flip their last bit likewise, plus where an h that differs moves
        them, well under 1%.  (A float32 BLAS evaluation of the same layer
        agrees with the oracle on 99.99% of h and 99.4% of the output.)  So h
        must equal the oracle's on at least 99.9% of elements and the output
        on at least 98%.
    """
    note("tp_mlp plain normal P=%d M=%d D=%d F=%d generate" % (P, M, D, F))
    x, w1, w2 = inputs.mlp_operands_normal(P, M, D, F, seed=675)
    note("tp_mlp plain normal P=%d M=%d D=%d F=%d run" % (P, M, D, F))
    gf, gh, go, _ = _run(x, w1, w2)
    np.testing.assert_array_equal(gf, np.stack([x.reshape(M, D)] * P))
    Mq = M // P
    note("tp_mlp plain normal check")
    _, h_ref, out_ref = oracle.tp_mlp_layer(x, w1, w2)
    for r in range(P):
        _, lo, hi, s, t = oracle.tp_mlp_bounds(x, w1, w2, r, np.arange(Mq))
        for q in range(P):
            hv = oracle.bf16_to_f32(gh[q][r * Mq:(r + 1) * Mq]).astype(np.float64)
            bad = ~((lo[q] <= hv) & (hv <= hi[q]))
            assert not bad.any(), "h of rank %d, rows of block %d: %d outside" % (q, r, int(bad.sum()))
        ov = oracle.bf16_to_f32(go[r]).astype(np.float64)
        bad = ~((oracle.bf16_nearest(s - t) <= ov) & (ov <= oracle.bf16_nearest(s + t)))
        assert not bad.any(), "out of rank %d: %d outside" % (r, int(bad.sum()))
    h_same = float(np.mean(gh == h_ref))
    o_same = float(np.mean(go == out_ref))
    print("h equal to the oracle's: %.5f, out equal: %.5f" % (h_same, o_same))
    assert h_same >= 0.999, h_same
    assert o_same >= 0.98, o_same


@pytest.mark.parametrize("P,M,D,F", [(16, 4096, 128, 2048), (32, 8192, 128, 4096)])
def test_many_ranks_integer_exact(P, M, D, F):
    """16 and 32 ranks, the fused path (one 256-row tile per rank): the
    gathered input, h and the output bit for bit."""
    note("tp_mlp many ranks P=%d M=%d D=%d F=%d" % (P, M, D, F))
    x, w1, w2 = _int_operands(P, M, D, F, seed=1440 + P)
    gf, gh, go, _ = _run(x, w1, w2)
    full, h, out = oracle.tp_mlp_layer(x, w1, w2)
    np.testing.assert_array_equal(gf, full)
    np.testing.assert_array_equal(gh, h)
    np.testing.assert_array_equal(go, out)


def test_single_layer_form_at_the_chapter_shape():
    """The chapter's single-layer form ends with an all-gather of the output
    shards (every device holds the layer's whole output): tp_mlp_layer, then
    ring_all_gather of its shards, at x [256, 1024], W1 [1024, 16384],
    W2 [16384, 1024], P = 4, on integer-valued operands; every rank's copy
    of the output bit for bit against the oracle's shards in rank order."""
    P, M, D, F = 4, 256, 1024, 16384
    note("tp_mlp single-layer form P=%d M=%d D=%d F=%d" % (P, M, D, F))
    x, w1, w2 = _int_operands(P, M, D, F, seed=650)
    _, _, go, ws = _run(x, w1, w2)
    Mq = M // P
    shards = [torch.from_numpy(np.ascontiguousarray(go[r]).view(np.int16)).cuda().view(torch.bfloat16)
              for r in range(P)]
    whole = [_nan_bf16((M * D,)) for _ in range(P)]
    ag_ws = rc.all_gather(whole, src=[s.reshape(-1) for s in shards])
    torch.cuda.synchronize()
    assert rc.last_error(ag_ws)[0] == 0
    _, _, out = oracle.tp_mlp_layer(x, w1, w2)
    want = out.reshape(P * Mq, D)
    for r in range(P):
        np.testing.assert_array_equal(whole[r].view(torch.int16).cpu().numpy().view(np.uint16).reshape(M, D), want)

"""Pins for the oracle's tensor-parallel MLP layer ("TPU 与分布式通信原语",
collective matmul: X = gelu(X @ W1) @ W2 with W1 split by columns and W2 by
rows; out_shard = ReduceScatter(gelu(AllGather(x_shard) @ W1_i) @ W2_i)).

What fixes it, other than the oracle itself:
  * gelu: PyTorch's own tanh-form gelu in fp64 where that form is accurate,
    the literal tanh formula in 80-digit decimal arithmetic in the tail, the
    odd-part identity gelu(x) - gelu(-x) = x, the Taylor coefficient
    1/sqrt(2 pi) at 0, and the distance to the exact GELU x Phi(x);
  * the bf16 roundings: torch's fp32 -> bf16 conversion on fp32 inputs, the
    double-rounding case fp64 -> fp32 -> bf16 gets wrong, directed roundings
    bracketing the value;
  * the layer: the unsharded single-device computation (one dense product
    per matrix), a pure-Python brute force on a tiny case, and the page's
    cost figures (2,147,483,648 flops per matmul at x [256, 1024], W1
    [1024, 16384], P = 4; 128 KiB shards, 384 KiB per direction).
"""
import decimal
import math

import numpy as np
import pytest
import torch

import oracle
from ring_collectives_amd import inputs


# ---------------------------------------------------------------- gelu
def test_gelu_matches_torch_tanh_form():
    x = np.linspace(-5.0, 10.0, 3001)
    want = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    got = oracle.gelu_tanh(x)
    mid = x >= -3.0
    np.testing.assert_allclose(got[mid], want[mid], rtol=1e-13, atol=1e-300)
    # torch's 1 + tanh(z) cancels for x < -3: still 1e-7 relative there
    np.testing.assert_allclose(got[~mid], want[~mid], rtol=1e-7)


def _gelu_decimal(x: float) -> float:
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) in 80 digits, tanh from
    its exponential definition."""
    with decimal.localcontext() as ctx:
        ctx.prec = 80
        X = decimal.Decimal(x)
        pi = decimal.Decimal("3.14159265358979323846264338327950288419716939937510582097494459")
        z = (2 / pi).sqrt() * (X + decimal.Decimal("0.044715") * X ** 3)
        e = (2 * z).exp()
        th = (e - 1) / (e + 1)
        return float(X * (1 + th) / 2)


@pytest.mark.parametrize("x", [-12.0, -10.5, -10.0, -8.0, -6.0, -4.0, -2.5, -0.75, 0.3, 1.0, 3.0, 7.5])
def test_gelu_against_decimal_literal_formula(x):
    want = _gelu_decimal(x)
    got = float(oracle.gelu_tanh(np.array([x]))[0])
    assert got == pytest.approx(want, rel=1e-13, abs=0.0), (x, got, want)


def test_gelu_identities():
    x = np.linspace(-6, 6, 1201)
    g = oracle.gelu_tanh
    # the tanh form's odd part is exactly x / 2
    np.testing.assert_allclose(g(x) - g(-x), x, rtol=0, atol=1e-14)
    assert g(np.array([0.0]))[0] == 0.0
    # gelu(x) = x/2 + x^2 / sqrt(2 pi) + O(x^4) (the tanh form keeps the slope
    # of the exact GELU at 0)
    for h in (1e-3, 1e-4):
        c = (g(np.array([h]))[0] - h / 2) / h ** 2
        assert c == pytest.approx(1 / math.sqrt(2 * math.pi), rel=1e-5)
    # an approximation of x Phi(x): close, but not equal
    from scipy.special import erf
    exact = 0.5 * x * (1 + erf(x / math.sqrt(2)))
    d = np.abs(g(x) - exact)
    assert d.max() < 1e-3 and d.max() > 1e-5


# ---------------------------------------------------------------- bf16
def test_bf16_from_f64_matches_torch_on_fp32_values():
    rng = np.random.default_rng(70)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))).astype(np.float32)
    v = np.concatenate([v, np.float32([0.0, -0.0, 1.00390625, 1.01171875, -1.00390625,
                                       2.0 ** -130, -3e-39, 1e-45])])
    want = inputs.bf16_bits(v)
    got = oracle.bf16_from_f64(v.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_from_f64_is_one_rounding():
    # 1 + 2^-8 + 2^-40 lies above the midpoint between 1 and 1 + 2^-7: one
    # rounding gives 1 + 2^-7; rounding to fp32 first lands on the midpoint
    # and then ties to even, 1.0
    v = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40, -(1.0 + 2.0 ** -8 + 2.0 ** -40)])
    np.testing.assert_array_equal(oracle.bf16_from_f64(v), np.array([0x3F81, 0xBF81], dtype=np.uint16))
    assert inputs.bf16_bits(v.astype(np.float32))[0] == 0x3F80


def test_nearest_is_monotone_and_within_half_a_step():
    rng = np.random.default_rng(71)
    v = np.sort(rng.standard_normal(20000) * np.exp2(rng.integers(-130, 100, 20000)))
    r = oracle.bf16_nearest(v)
    assert np.all(np.diff(r) >= 0)
    np.testing.assert_array_equal(r, oracle.bf16_to_f32(oracle.bf16_from_f64(v)).astype(np.float64))
    _, e = np.frexp(v)
    half = np.ldexp(1.0, np.maximum(e, -125) - 9)
    assert np.all(np.abs(r - v) <= half)
    np.testing.assert_array_equal(oracle.bf16_nearest(r), r)   # bf16 values are fixed points


# ---------------------------------------------------------------- the layer
def _dense(x_shards, W1, W2):
    """Single device: X = concat of the row blocks, W1 = concat of the column
    blocks, W2 = concat of the row blocks; one product per matrix."""
    P, Mq, D = x_shards.shape
    f = lambda a: oracle.bf16_to_f32(a).astype(np.float64)
    X = f(x_shards.reshape(P * Mq, D))
    w1 = np.concatenate([f(W1[q]) for q in range(P)], axis=1)
    w2 = np.concatenate([f(W2[q]) for q in range(P)], axis=0)
    h = oracle.bf16_from_f64(oracle.gelu_tanh(f(oracle.bf16_from_f64(X @ w1))))
    return h, f(h) @ w2


@pytest.mark.parametrize("P", [1, 2, 3, 4])
def test_layer_equals_unsharded_computation(P):
    Mq, D, F = 16, 64, 32 * P
    x, w1, w2 = inputs.mlp_operands(P, Mq * P, D, F, seed=72 + P)
    full, h, out = oracle.tp_mlp_layer(x, w1, w2)
    h_dense, y = _dense(x, w1, w2)
    Fr = F // P
    for q in range(P):
        np.testing.assert_array_equal(full[q], x.reshape(P * Mq, D))
        np.testing.assert_array_equal(h[q], h_dense[:, q * Fr:(q + 1) * Fr])
    got = oracle.bf16_to_f32(out.reshape(P * Mq, D)).astype(np.float64)
    mag = np.abs(oracle.bf16_to_f32(h_dense).astype(np.float64)) @ np.abs(
        np.concatenate([oracle.bf16_to_f32(w2[q]) for q in range(P)], axis=0).astype(np.float64))
    # one bf16 rounding of an fp32 sum within the recursive-summation bound
    assert np.all(np.abs(got - y) <= 2.0 ** -8 * np.abs(y) + (Fr + P) * 2.0 ** -24 * mag * 1.01)
    # rank r owns row block r
    assert not np.array_equal(out[0], out[-1]) or P == 1


def test_layer_brute_force_tiny():
    """P = 2, M = 2, D = 2, F = 4, integer-valued data: every step with
    Python scalars (the tanh formula written out), every bit equal."""
    P, D, Fr = 2, 2, 2
    xs = [[[1.0, 2.0]], [[-1.0, 3.0]]]                  # rank q's row
    W1 = [[[1.0, 0.0], [1.0, -1.0]], [[0.0, 2.0], [-1.0, 1.0]]]
    W2 = [[[1.0, -2.0], [3.0, 1.0]], [[-1.0, 1.0], [2.0, 2.0]]]
    X = [xs[0][0], xs[1][0]]

    def bf(v):
        return int(inputs.bf16_bits(np.float32([v]))[0])

    def bfval(b):
        return float(oracle.bf16_to_f32(np.array([b], dtype=np.uint16))[0])

    def gelu(v):
        return 0.5 * v * (1.0 + math.tanh(math.sqrt(2 / math.pi) * (v + 0.044715 * v ** 3)))

    h = [[[0] * Fr for _ in range(2)] for _ in range(P)]
    for q in range(P):
        for i in range(2):
            for j in range(Fr):
                a = sum(X[i][k] * W1[q][k][j] for k in range(D))
                h[q][i][j] = bf(gelu(bfval(bf(a))))
    y = [[sum(bfval(h[q][i][k]) * W2[q][k][j] for q in range(P) for k in range(Fr)) for j in range(D)]
         for i in range(2)]
    want = np.array([[[bf(y[r][j]) for j in range(D)]] for r in range(P)], dtype=np.uint16)
    arr = lambda v: inputs.bf16_bits(np.array(v, dtype=np.float32))
    _, hh, out = oracle.tp_mlp_layer(arr(xs), arr(W1), arr(W2))
    np.testing.assert_array_equal(hh, np.array(h, dtype=np.uint16))
    np.testing.assert_array_equal(out, want)


def test_first_product_exact_on_the_grid_inputs():
    """The workload's x and W1 sit on grids 2^-4 and 2^-10, so x @ W1 is
    exact in fp32 in any order; the bounds then give h one value almost
    everywhere."""
    P, M, D, F = 2, 64, 1024, 256
    x, w1, w2 = inputs.mlp_operands(P, M, D, F, seed=80)
    X = oracle.bf16_to_f32(x.reshape(M, D)).astype(np.float64)
    assert oracle._exact_in_fp32(X, oracle.bf16_to_f32(w1[0]).astype(np.float64))
    h_ref, lo, hi, s, t = oracle.tp_mlp_bounds(x, w1, w2, 0, np.arange(M // P))
    ref = oracle.bf16_to_f32(h_ref).astype(np.float64)
    assert np.all((lo <= ref) & (ref <= hi))
    assert np.mean(lo != hi) < 0.01
    # the oracle's own output lies in its interval
    _, _, out = oracle.tp_mlp_layer(x, w1, w2)
    got = oracle.bf16_to_f32(out[0]).astype(np.float64)
    assert np.all((oracle.bf16_nearest(s - t) <= got) & (got <= oracle.bf16_nearest(s + t)))
    # and the interval is narrow: about one bf16 step
    assert np.median(t / np.maximum(np.abs(s), 1e-30)) < 2.0 ** -10


def test_bounds_widen_when_the_product_is_not_exact():
    P, M, D, F = 2, 32, 128, 256
    rng = np.random.default_rng(81)
    x = inputs.bf16_bits(rng.standard_normal((P, M // P, D)).astype(np.float32))
    w1 = inputs.bf16_bits((rng.standard_normal((P, D, F // P)) / 11).astype(np.float32))
    w2 = inputs.bf16_bits((rng.standard_normal((P, F // P, D)) / 16).astype(np.float32))
    X = oracle.bf16_to_f32(x.reshape(M, D)).astype(np.float64)
    assert not oracle._exact_in_fp32(X, oracle.bf16_to_f32(w1[0]).astype(np.float64))
    _, lo, hi, _, _ = oracle.tp_mlp_bounds(x, w1, w2, 1, np.arange(M // P))
    assert np.mean(lo != hi) > 0.05


def test_page_cost_figures():
    """x [256, 1024], W1 [1024, 16384], W2 [16384, 1024], 4 devices: each
    device's all-gather-matmul and matmul-reduce-scatter take
    2 * 256 * 1024 * 4096 = 2,147,483,648 flops; a shard is 128 KiB and a
    device sends 3 of them, 384 KiB, in one direction."""
    import bench
    f = bench.mlp_layer_cost(P=4, M=256, D=1024, F=16384)
    assert f["flop_per_matmul_per_rank"] == 2147483648
    assert f["flop"] == 4 * 2 * 2147483648
    assert f["shard_bytes"] == 131072
    assert f["ring_bytes_per_direction"] == 3 * 131072


# ---------------------------------------------------------------- gelu's fp32 allowance
def _every_finite_bf16():
    u = np.arange(65536, dtype=np.uint32)
    return u[((u >> 7) & 0xFF) != 255].astype(np.uint16)


@pytest.fixture(scope="module")
def gelu_intervals():
    """The oracle's interval for h = bf16(gelu(b)) at every finite bf16 b, as
    tp_mlp_bounds gives it for a layer whose first product is exactly b
    (x rows are unit vectors, W1 holds the values)."""
    vals = _every_finite_bf16()
    D = F = 256
    w1 = np.concatenate([vals, vals[:D * F - len(vals)]]).reshape(1, D, F)
    x = np.zeros((1, 256, D), dtype=np.float32)
    x[0, np.arange(256), np.arange(256)] = 1.0
    _, lo, hi, _, _ = oracle.tp_mlp_bounds(inputs.bf16_bits(x), w1, np.zeros((1, F, D), np.uint16), 0,
                                           np.arange(256))
    n = len(vals)
    b = (vals.astype(np.uint32) << 16).view(np.float32)
    return b, lo[0].reshape(-1)[:n], hi[0].reshape(-1)[:n]


def _bf16_of(g32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's conversion, nearest-even) as fp64 values."""
    return torch.from_numpy(np.ascontiguousarray(g32, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _gelu_f32_tanh(b, c=np.sqrt(2.0 / np.pi), k=0.044715):
    """The page's formula, 0.5 x (1 + tanh(c (x + k x^3))), in NumPy float32."""
    c, k = np.float32(c), np.float32(k)
    with np.errstate(over="ignore", invalid="ignore"):
        z = c * (b + k * b * b * b)
        return np.float32(0.5) * b * (np.float32(1.0) + np.tanh(z)), np.float32(1.0) + np.tanh(z)


def _gelu_f32_logistic(b, c=np.sqrt(2.0 / np.pi), k=0.044715, split=True):
    """x sigmoid(2z) in NumPy float32 through e = exp(-|2z|) <= 1:
    x / (1 + e) for x >= 0, x e / (1 + e) for x < 0 (split=False: the first
    form everywhere)."""
    c, k = np.float32(c), np.float32(k)
    with np.errstate(over="ignore", invalid="ignore"):
        t = np.float32(2.0) * c * (b + k * b * b * b)
        e = np.exp(-np.abs(t))
        pos = b / (np.float32(1.0) + e)
        neg = b * e / (np.float32(1.0) + e)
        return np.where(b >= 0, pos, neg) if split else b / (np.float32(1.0) + np.exp(-t))


def _inside(h, lo, hi):
    return (lo <= h) & (h <= hi)


def test_gelu_intervals_are_tight(gelu_intervals):
    """One admissible h on at least 99% of all finite bf16 inputs (what is
    left is mostly subnormal inputs whose gelu, x/2 to within 1e-40 relative,
    sits on a bf16 rounding tie)."""
    _, lo, hi = gelu_intervals
    assert np.mean(lo == hi) >= 0.99, np.mean(lo == hi)


def test_independent_fp32_gelu_lands_inside(gelu_intervals):
    """Plain fp32 evaluations written apart from the oracle and the kernel
    land inside the intervals: the logistic form everywhere; the page's tanh
    form, in NumPy float32 and as torch's float32 gelu, wherever 1 + tanh z
    holds at least 1/16 (further left it cancels and loses the relative
    accuracy the bound is about: the reason an implementation evaluates the
    logistic)."""
    b, lo, hi = gelu_intervals
    assert _inside(_bf16_of(_gelu_f32_logistic(b)), lo, hi).all()
    g_tanh, one_plus = _gelu_f32_tanh(b)
    ok = one_plus >= np.float32(1.0 / 16)
    assert ok[b >= -1.8].all() and ok.sum() > 0.7 * len(b)  # all x >= -1.8 (3/4 of the bf16 values)
    assert _inside(_bf16_of(g_tanh), lo, hi)[ok].all()
    g_torch = torch.nn.functional.gelu(torch.from_numpy(b), approximate="tanh").numpy()
    assert _inside(_bf16_of(g_torch), lo, hi)[ok].all()


@pytest.mark.parametrize("mistake", ["k=0.04472", "c=sqrt(1/pi)", "no cube", "one branch", "tanh unguarded"])
def test_plausible_gelu_mistakes_fall_outside(gelu_intervals, mistake):
    """Each plausible slip in an fp32 gelu puts results outside the
    intervals on some inputs: the intervals are tight enough to catch it."""
    b, lo, hi = gelu_intervals
    if mistake == "k=0.04472":
        g = _gelu_f32_logistic(b, k=0.04472)
    elif mistake == "c=sqrt(1/pi)":
        g = _gelu_f32_logistic(b, c=np.sqrt(1.0 / np.pi))
    elif mistake == "no cube":
        g = _gelu_f32_logistic(b, k=0.0)
    elif mistake == "one branch":                             # x / (1 + exp(-t)) overflows for x < -10
        g = _gelu_f32_logistic(b, split=False)
    else:                                                   # the tanh form where it cancels
        g = _gelu_f32_tanh(b)[0]
    assert (~_inside(_bf16_of(g), lo, hi)).sum() >= 5

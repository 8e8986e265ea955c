"""Pins for the oracle's bidirectional reduce-scatter ("Pallas TPU Distributed
Collectives 复习文档", section 4: lax.psum_scatter with the top half of every
block travelling left and the bottom half right).

What fixes it, other than the oracle itself:
  * the page's P = 4 walk-through (section 4.6): for every step and phase the
    table names the block a device accumulates and the devices whose
    contributions it holds, in the order they were added; the fixture
    tests/golden/bidir_rs_p4_trace.txt transcribes it and the test evaluates
    each entry in fp32 in that order, on data whose rounding depends on it;
  * the semantics of section 4.4 (device d ends with the sum over devices of
    block d), checked by brute force on integers;
  * the contributor set of every partial sum, with one bit per rank;
  * the error bound of recursive summation.
"""
import os

import numpy as np
import pytest

import oracle
from ring_collectives_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PS = [1, 2, 3, 4, 5, 8, 16]


def _trace_rows():
    rows = []
    with open(os.path.join(GOLDEN, "bidir_rs_p4_trace.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            step, phase, dev, block, half, order = line.split()
            rows.append((int(step), phase, int(dev), int(block), half,
                         [int(q) for q in order.split("+")]))
    return rows


def _half(C, half):
    h = oracle.bidir_top_len(C)
    return slice(0, h) if half == "T" else slice(h, C)


def _wide_f32(P, n, seed):
    """fp32 values spread over 40 binades, so the order of additions shows in
    the rounded bits."""
    rng = np.random.default_rng(seed)
    m = rng.standard_normal((P, n)).astype(np.float32)
    e = rng.integers(-20, 20, size=(P, n)).astype(np.float32)
    return (m * np.exp2(e)).astype(np.float32)


def test_trace_fixture_is_complete():
    rows = _trace_rows()
    assert len(rows) == 4 * 2 * 4
    # every (step, phase, device) appears once; the last step holds block d
    assert len({(s, ph, d) for s, ph, d, _, _, _ in rows}) == 32
    for s, ph, d, b, half, order in rows:
        assert (ph == "L") == (half == "T")
        assert order[0] == b and len(order) == min(s + 2, 4)
        if s == 3:
            assert b == d


def test_bidir_matches_page_trace_in_fp32_order():
    P, C = 4, 64
    x = _wide_f32(P, P * C, seed=40)
    states = [oracle.reduce_scatter_bidir(x, steps=s + 1) for s in range(P)]
    for s, ph, d, b, half, order in _trace_rows():
        sl = _half(C, half)
        want = x[order[0], b * C:(b + 1) * C][sl].copy()
        for q in order[1:]:
            want = (want + x[q, b * C:(b + 1) * C][sl]).astype(np.float32)
        got = states[s][d, b * C:(b + 1) * C][sl]
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32),
                                      err_msg="step %d %s device %d" % (s, ph, d))


def test_page_trace_order_is_discriminating():
    """On the same data another order of the same contributors gives other
    bits, so the previous test pins the order and not only the set."""
    P, C = 4, 64
    x = _wide_f32(P, P * C, seed=40)
    differs = 0
    for s, ph, d, b, half, order in _trace_rows():
        if len(order) < 3:
            continue
        sl = _half(C, half)
        a = x[order[0], b * C:(b + 1) * C][sl].copy()
        for q in order[1:]:
            a = (a + x[q, b * C:(b + 1) * C][sl]).astype(np.float32)
        rev = x[order[-1], b * C:(b + 1) * C][sl].copy()
        for q in order[-2::-1]:
            rev = (rev + x[q, b * C:(b + 1) * C][sl]).astype(np.float32)
        differs += int(np.any(a.view(np.uint32) != rev.view(np.uint32)))
    assert differs >= 16


@pytest.mark.parametrize("P", PS)
def test_bidir_is_psum_scatter_int32(P):
    """Section 4.4: device d ends with the sum over devices of block d."""
    x = inputs.to_chunk_major(inputs.ring_i32(P), P)
    st = oracle.reduce_scatter_bidir(x)
    C = x.shape[1] // P
    want = x.astype(np.int64).sum(axis=0).astype(np.int32)
    for d in range(P):
        np.testing.assert_array_equal(st[d, d * C:(d + 1) * C], want[d * C:(d + 1) * C])


@pytest.mark.parametrize("P", [2, 3, 4, 5, 8, 16])
def test_bidir_contributor_sets(P):
    """One bit per rank: after step s the top half of chunk (d+s+1) holds the
    ranks d+s+1 down to d and the bottom half of chunk (d-s-1) the ranks
    d-s-1 up to d (the halves' routes in section 4.2's figure)."""
    C = 6
    x = np.repeat((1 << np.arange(P, dtype=np.int64)).astype(np.int32)[:, None], P * C, axis=1)
    h = oracle.bidir_top_len(C)
    for s in range(P - 1):
        st = oracle.reduce_scatter_bidir(x, steps=s + 1)
        for d in range(P):
            ct, cb = (d + s + 1) % P, (d - s - 1) % P
            top = sum(1 << ((d + i) % P) for i in range(s + 2))
            bot = sum(1 << ((d - i) % P) for i in range(s + 2))
            assert np.all(st[d, ct * C:ct * C + h] == top), (P, s, d)
            assert np.all(st[d, cb * C + h:(cb + 1) * C] == bot), (P, s, d)


@pytest.mark.parametrize("P,C", [(3, 5), (4, 1), (5, 7), (2, 3)])
def test_bidir_odd_chunks(P, C):
    """A chunk of odd length splits into C - C//2 top and C//2 bottom
    elements; the result is still the sum over ranks."""
    rng = np.random.default_rng(41 + P)
    x = rng.integers(-1000, 1000, size=(P, P * C), endpoint=True).astype(np.int32)
    st = oracle.reduce_scatter_bidir(x)
    want = x.astype(np.int64).sum(axis=0)
    for d in range(P):
        np.testing.assert_array_equal(st[d, d * C:(d + 1) * C].astype(np.int64),
                                      want[d * C:(d + 1) * C])


def test_bidir_p1_identity_and_p2():
    x = inputs.small_f32(1).reshape(1, -1)
    np.testing.assert_array_equal(oracle.reduce_scatter_bidir(x), x)
    # P = 2: device 0's block 0 is x0 + x1 in both halves (each half starts
    # at its owner and takes one more contribution)
    x = _wide_f32(2, 2 * 16, seed=42)
    st = oracle.reduce_scatter_bidir(x)
    want = (x[0] + x[1]).astype(np.float32)
    np.testing.assert_array_equal(st[0, :16].view(np.uint32), want[:16].view(np.uint32))
    np.testing.assert_array_equal(st[1, 16:].view(np.uint32), want[16:].view(np.uint32))


@pytest.mark.parametrize("P", [2, 4, 8, 16])
def test_bidir_fp32_within_recursive_sum_bound(P):
    x = inputs.normal_f32(P, 1024 * P, seed=43)
    st = oracle.reduce_scatter_bidir(x)
    ref, mag = oracle.rank_sum_f64(x)
    C = x.shape[1] // P
    worst = 0.0
    for d in range(P):
        sl = slice(d * C, (d + 1) * C)
        err = np.abs(st[d, sl].astype(np.float64) - ref[sl]) / np.maximum(mag[sl], 1e-300)
        worst = max(worst, float(err.max()))
    assert worst <= (P - 1) * 2.0 ** -24 * (1 + 1e-6)


def test_bidir_order_differs_from_one_way_ring():
    """Owner first (bidirectional) against owner last (one-way ring): same
    sums, different association, so different bits somewhere."""
    P = 4
    x = _wide_f32(P, P * 64, seed=44)
    a = oracle.reduce_scatter_bidir(x)
    b = oracle.reduce_scatter(x)
    C = 64
    assert any(np.any(a[d, d * C:(d + 1) * C].view(np.uint32) != b[d, d * C:(d + 1) * C].view(np.uint32))
               for d in range(P))


@pytest.mark.parametrize("P", [2, 4, 16])
def test_bidir_bf16_one_rounding(P):
    """fp32 halves, one rounding of the complete block: the bf16 result is
    the rounding of the fp32 schedule run on the widened inputs, and lies
    within 2^-8 |sum| + (P-1) 2^-24 sum|x| of the exact sum."""
    x = inputs.normal_bf16(P, 512 * P, seed=45)
    dst, carry = oracle.reduce_scatter_bidir_bf16(x)
    wide = oracle.reduce_scatter_bidir(oracle.bf16_to_f32(x).copy())
    np.testing.assert_array_equal(carry.view(np.uint32), wide.view(np.uint32))
    C = x.shape[1] // P
    ref, mag = oracle.rank_sum_f64(x, bf16=True)
    for d in range(P):
        sl = slice(d * C, (d + 1) * C)
        np.testing.assert_array_equal(dst[d, sl], oracle.bf16_from_f32(wide[d, sl]))
        got = oracle.bf16_to_f32(dst[d, sl]).astype(np.float64)
        err = np.abs(got - ref[sl]) / np.maximum(mag[sl], 1e-300)
        assert err.max() <= 2.0 ** -8 + (P - 1) * 2.0 ** -24 + 1e-9

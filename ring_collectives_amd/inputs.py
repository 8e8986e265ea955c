"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and lays them out; it holds none of the
collectives' arithmetic.  Everything is NumPy PCG64:
  * small workloads: ``default_rng(seed)``, one draw of shape (P, ...) in rank
    order;
  * large workloads (fp32/bf16 normal rank buffers, GEMM operands): rank r
    draws from its own child stream ``default_rng(SeedSequence(seed).spawn(P)[r])``
    so the ranks can be drawn in parallel threads; bf16 data is drawn in
    slabs, which continue the same per-rank stream.

bf16 values are the round-to-nearest-even images of fp32 draws, produced with
torch's fp32 -> bf16 conversion and handled here as uint16 bit patterns.

Workloads (the pages draw their inputs with JAX keys that cannot be replayed
here, so only shape, type and distribution follow them):
  * small fp32 ring: P ranks, each an fp32 (8, 512) array, uniform [0, 1),
    seed 0 -- the (8, 128 * devices) shape of "Pallas TPU Distributed
    Collectives 复习文档" section 1.3 at four devices;
  * int32 ring: P ranks, each int32 (8, 128 * P), uniform integers in
    [-1000, 1000], seed 1;
  * fp32 bandwidth workload: P = 8, 64 Mi fp32 per rank, normal(0, 1), seed 2;
  * bf16 gradient-bucket workload: P = 16, 128 Mi bf16 per rank,
    normal(0, 0.01), seed 3;
  * GEMM + reduce-scatter: P = 4, A_q and B_q bf16 4096 x 4096,
    normal(0, 1/64), seed 4 (all-gather + GEMM: the same shapes, seed 5);
  * tensor-parallel MLP layer: P = 4, x [M, 1024], W1 [1024, 16384],
    W2 [16384, 1024], seed 6: plain normal bf16 operands (mlp_operands_normal)
    and operands on fixed-point grids whose first product is exact
    (mlp_operands).

Two-dimensional per-rank arrays of shape (R, w * P) are stored chunk-major:
chunk c (a flat, contiguous run of R * w elements) is column block c of the
logical array, as in the chunk-major layout helpers of "TPU 与分布式通信原语"
(collective matmul section).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED_SMALL_F32 = 0
SEED_I32 = 1
SEED_F32_BW = 2
SEED_BF16 = 3
SEED_GEMM = 4


# ---------------------------------------------------------------- layout
def to_chunk_major(x: np.ndarray, P: int) -> np.ndarray:
    """(ranks, R, w*P) logical arrays -> (ranks, P*R*w) flat chunk-major."""
    ranks, R, W = x.shape
    w = W // P
    return np.ascontiguousarray(x.reshape(ranks, R, P, w).transpose(0, 2, 1, 3)).reshape(ranks, -1)


def from_chunk_major(flat: np.ndarray, P: int, R: int) -> np.ndarray:
    """(ranks, P*R*w) chunk-major -> (ranks, R, w*P) logical arrays."""
    ranks = flat.shape[0]
    w = flat.shape[1] // (P * R)
    return np.ascontiguousarray(flat.reshape(ranks, P, R, w).transpose(0, 2, 1, 3)).reshape(ranks, R, P * w)


def bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 (RNE) as uint16 bit patterns, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- workloads
def small_f32(P: int, shape=(8, 512)) -> np.ndarray:
    """Logical per-rank fp32 arrays, uniform [0, 1), seed 0 -> (P, R, W)."""
    rng = np.random.default_rng(SEED_SMALL_F32)
    return rng.random((P, *shape), dtype=np.float32)


def ring_i32(P: int, rows: int = 8, width_per_rank: int = 128) -> np.ndarray:
    """Logical per-rank int32 arrays (rows, width_per_rank * P), uniform
    integers in [-1000, 1000], seed 1 -> (P, rows, width_per_rank * P)."""
    rng = np.random.default_rng(SEED_I32)
    return rng.integers(-1000, 1000, size=(P, rows, width_per_rank * P),
                        endpoint=True, dtype=np.int32)


def rank_streams(seed: int, P: int):
    """One independent PCG64 generator per rank, spawned from `seed`."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(P)]


def _threads(P: int) -> int:
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:
        cpus = os.cpu_count() or 1
    return max(1, min(P, cpus, 16))


def normal_f32(P: int, n: int, seed: int = SEED_F32_BW, std: float = 1.0) -> np.ndarray:
    """(P, n) fp32 normal(0, std); rank r from its own child stream."""
    out = np.empty((P, n), dtype=np.float32)
    gens = rank_streams(seed, P)

    def draw(r):
        gens[r].standard_normal(n, dtype=np.float32, out=out[r])
        if std != 1.0:
            out[r] *= np.float32(std)

    with ThreadPoolExecutor(_threads(P)) as ex:
        list(ex.map(draw, range(P)))
    return out


def normal_bf16(P: int, n: int, seed: int = SEED_BF16, std: float = 1e-2,
                slab: int = 1 << 24) -> np.ndarray:
    """(P, n) bf16 bit patterns: RNE of fp32 normal(0, std) draws; rank r
    from its own child stream, drawn in slabs of `slab` values."""
    out = np.empty((P, n), dtype=np.uint16)
    gens = rank_streams(seed, P)

    def draw(r):
        buf = np.empty(min(slab, max(n, 1)), dtype=np.float32)
        for lo in range(0, n, slab):
            m = min(slab, n - lo)
            gens[r].standard_normal(m, dtype=np.float32, out=buf[:m])
            buf[:m] *= np.float32(std)
            out[r, lo:lo + m] = bf16_bits(buf[:m])

    with ThreadPoolExecutor(_threads(P)) as ex:
        list(ex.map(draw, range(P)))
    return out


def gemm_operands(P: int = 4, M: int = 4096, N: int = 4096, K: int = 4096,
                  std: float = 1.0 / 64, seed: int = SEED_GEMM):
    """(A, B) as bf16 bit patterns: A (P, M, K), B (P, K, N), normal(0, std).
    Rank q draws A_q and then B_q from its own child stream."""
    A = np.empty((P, M, K), dtype=np.uint16)
    B = np.empty((P, K, N), dtype=np.uint16)
    gens = rank_streams(seed, P)

    def draw(q):
        a = gens[q].standard_normal((M, K), dtype=np.float32) * np.float32(std)
        A[q] = bf16_bits(a)
        b = gens[q].standard_normal((K, N), dtype=np.float32) * np.float32(std)
        B[q] = bf16_bits(b)

    with ThreadPoolExecutor(_threads(P)) as ex:
        list(ex.map(draw, range(P)))
    return A, B


def small_int_bf16(rng: np.random.Generator, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Integer-valued bf16 bit patterns (uniform integers in [lo, hi]); every
    such value is exact in bf16."""
    return bf16_bits(rng.integers(lo, hi, size=shape, endpoint=True).astype(np.float32))


SEED_MLP = 6


def mlp_operands(P: int = 4, M: int = 8192, D: int = 1024, F: int = 16384, seed: int = SEED_MLP):
    """Tensor-parallel MLP layer operands as bf16 bit patterns: the layer
    input's row blocks x (P, M/P, D), the column blocks of W1 (P, D, F/P) and
    the row blocks of W2 (P, F/P, D) -- the x [tokens, 1024], W1 [1024, 16384],
    W2 [16384, 1024] shapes of "TPU 与分布式通信原语" (collective matmul) at
    P = 4, with more tokens.

    x is normal(0, 1) on the grid 2^-4 (clipped to [-4, 4]) and W1 normal(0,
    1/D) on the grid 2^-10 (clipped to 127 steps), so every product x w is a
    multiple of 2^-14 and, for D up to 2048, every partial sum of x @ W1 is
    exact in fp32 whatever the order; W2 is normal(0, 1/F) rounded to bf16.
    Rank q draws x_q, W1_q and W2_q, in that order, from its own child stream.
    """
    Mq, Fr = M // P, F // P
    x = np.empty((P, Mq, D), dtype=np.uint16)
    w1 = np.empty((P, D, Fr), dtype=np.uint16)
    w2 = np.empty((P, Fr, D), dtype=np.uint16)
    gens = rank_streams(seed, P)

    def draw(q):
        g = gens[q]
        a = np.clip(np.rint(g.standard_normal((Mq, D), dtype=np.float32) * 16.0), -64, 64)
        x[q] = bf16_bits((a / 16.0).astype(np.float32))
        b = np.clip(np.rint(g.standard_normal((D, Fr), dtype=np.float32) * (1024.0 / np.sqrt(D))),
                    -127, 127)
        w1[q] = bf16_bits((b / 1024.0).astype(np.float32))
        c = g.standard_normal((Fr, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(F))
        w2[q] = bf16_bits(c)

    with ThreadPoolExecutor(_threads(P)) as ex:
        list(ex.map(draw, range(P)))
    return x, w1, w2


def mlp_operands_normal(P: int = 4, M: int = 8192, D: int = 1024, F: int = 16384, seed: int = SEED_MLP):
    """Tensor-parallel MLP layer operands as bf16 bit patterns, shaped as in
    mlp_operands, with plain normal values rounded to bf16 (nearest even):
    x normal(0, 1), W1 normal(0, 1/D), W2 normal(0, 1/F) -- the scale of an
    initialised layer.  Rank q draws x_q, W1_q and W2_q, in that order, from
    its own child stream."""
    Mq, Fr = M // P, F // P
    x = np.empty((P, Mq, D), dtype=np.uint16)
    w1 = np.empty((P, D, Fr), dtype=np.uint16)
    w2 = np.empty((P, Fr, D), dtype=np.uint16)
    gens = rank_streams(seed, P)

    def draw(q):
        g = gens[q]
        x[q] = bf16_bits(g.standard_normal((Mq, D), dtype=np.float32))
        w1[q] = bf16_bits(g.standard_normal((D, Fr), dtype=np.float32) * np.float32(1.0 / np.sqrt(D)))
        w2[q] = bf16_bits(g.standard_normal((Fr, D), dtype=np.float32) * np.float32(1.0 / np.sqrt(F)))

    with ThreadPoolExecutor(_threads(P)) as ex:
        list(ex.map(draw, range(P)))
    return x, w1, w2

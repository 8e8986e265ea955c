"""CPU oracle for the ring collectives -- TEST INFRASTRUCTURE ONLY.

This package is the yardstick the GPU library is checked against.  It is
plain, slow and single-threaded on purpose, shares no code with the GPU path
and never imports it.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product path must never
route through it.

The ring arithmetic lives in ``ring_oracle.c`` (plain C, built with
``-ffp-contract=off`` and without fast-math so every fp32 addition is one
IEEE-754 round-to-nearest-even addition).  This module loads it with ctypes
and wraps it for NumPy arrays shaped ``(P, n)`` (rank-major, rank r in row r).

The GEMM part of the GEMM + reduce-scatter oracle uses NumPy's float64 matrix
product as a library step (products of bf16 values are exact in fp64; the
4096-term sums carry ~1e-16 relative error), rounds once to fp32, and then runs
the same fp32 ring reduce-scatter as the collectives.

Sources followed (page title, section):
  * "Pallas TPU Distributed Collectives 复习文档": 0.1 ring model, 1 right
    shift (ppermute), 2 all_gather, 4.4 psum_scatter semantics.
  * "TPU 与分布式通信原语": reduce-scatter / all-gather ring kernels;
    collective matmul (matmul then reduce-scatter over row blocks).
  * "全归约 3：Ring——每步大小恒定": The idea; Walkthrough (index arithmetic,
    one signal row per round); Edge cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ring_oracle.c")
_LIB = os.path.join(_HERE, "libring_oracle.so")

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fno-unsafe-math-optimizations", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile ring_oracle.c with gcc into libring_oracle.so (in place)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        for name, args in {
            "oracle_ppermute": [vp, vp, i32, sz],
            "oracle_reduce_scatter_f32": [vp, vp, i32, sz, i32],
            "oracle_reduce_scatter_i32": [vp, vp, i32, sz, i32],
            "oracle_all_gather": [vp, i32, sz, sz, i32],
            "oracle_all_gather_place": [vp, vp, i32, sz, sz],
            "oracle_all_reduce_f32": [vp, vp, i32, sz],
            "oracle_all_reduce_i32": [vp, vp, i32, sz],
            "oracle_reduce_scatter_bf16": [vp, vp, vp, i32, sz, i32],
            "oracle_all_reduce_bf16": [vp, vp, vp, i32, sz],
            "oracle_reduce_scatter_bidir_f32": [vp, vp, i32, sz, i32],
            "oracle_reduce_scatter_bidir_i32": [vp, vp, i32, sz, i32],
            "oracle_reduce_scatter_bidir_bf16": [vp, vp, vp, i32, sz, i32],
            "oracle_psum_circ_f32": [vp, vp, vp, i32, sz, i32],
            "oracle_psum_circ_i32": [vp, vp, vp, i32, sz, i32],
            "oracle_psum_circ_bf16": [vp, vp, i32, sz],
            "oracle_bf16_from_f32_array": [vp, vp, sz],
            "oracle_rank_sum_f64_f32": [vp, i32, sz, vp, vp],
            "oracle_rank_sum_f64_bf16": [vp, i32, sz, vp, vp],
        }.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        lib.oracle_bf16_from_f32_array.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError("oracle: invalid arguments to %s" % what)


def _ranks(x: np.ndarray, dtype) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != dtype or x.ndim < 2:
        raise TypeError("expected a (P, ...) array of %s, got %s %s" % (dtype, x.dtype, x.shape))
    return x


# --------------------------------------------------------------------------
# collectives on (P, n) arrays
# --------------------------------------------------------------------------
def ppermute(x: np.ndarray) -> np.ndarray:
    """Right shift: out[r] = x[left(r)] (every rank sends its buffer right)."""
    x = np.ascontiguousarray(x)
    P = x.shape[0]
    out = np.empty_like(x)
    _check(_load().oracle_ppermute(_ptr(x), _ptr(out), P, x[0].nbytes), "ppermute")
    return out


def reduce_scatter(x: np.ndarray, rounds: int | None = None) -> np.ndarray:
    """Ring reduce-scatter state after `rounds` rounds (default P-1).

    fp32 and int32 inputs.  Returns the whole (P, n) state; after all P-1
    rounds chunk r of row r is the sum over ranks (the other chunks hold
    partial sums)."""
    x = np.ascontiguousarray(x)
    P = x.shape[0]
    n = x[0].size
    rounds = P - 1 if rounds is None else rounds
    out = np.empty_like(x)
    lib = _load()
    if x.dtype == np.float32:
        rc = lib.oracle_reduce_scatter_f32(_ptr(x), _ptr(out), P, n, rounds)
    elif x.dtype == np.int32:
        rc = lib.oracle_reduce_scatter_i32(_ptr(x), _ptr(out), P, n, rounds)
    else:
        raise TypeError("reduce_scatter: fp32 or int32 (bf16: reduce_scatter_bf16)")
    _check(rc, "reduce_scatter")
    return out


def bidir_top_len(C: int) -> int:
    """Elements in the top half of a chunk of C elements (the half that
    travels left in the bidirectional reduce-scatter)."""
    return C - C // 2


def reduce_scatter_bidir(x: np.ndarray, steps: int | None = None) -> np.ndarray:
    """Bidirectional ring reduce-scatter ("Pallas TPU Distributed Collectives
    复习文档" section 4): top halves of the chunks travel left, bottom halves
    right, each summed owner first.  fp32 and int32.  Returns the (P, n)
    state after `steps` steps (default P): the sum computed at step s sits at
    the top half of chunk (d+s+1) mod P and the bottom half of chunk
    (d-s-1) mod P of row d; after all P steps chunk d of row d is the sum
    over ranks."""
    x = np.ascontiguousarray(x)
    P = x.shape[0]
    n = x[0].size
    steps = P if steps is None else steps
    out = np.empty_like(x)
    lib = _load()
    if x.dtype == np.float32:
        rc = lib.oracle_reduce_scatter_bidir_f32(_ptr(x), _ptr(out), P, n, steps)
    elif x.dtype == np.int32:
        rc = lib.oracle_reduce_scatter_bidir_i32(_ptr(x), _ptr(out), P, n, steps)
    else:
        raise TypeError("reduce_scatter_bidir: fp32 or int32 (bf16: reduce_scatter_bidir_bf16)")
    _check(rc, "reduce_scatter_bidir")
    return out


def psum_circulating(x: np.ndarray, steps: int | None = None):
    """Circulating-input psum ("Pallas TPU Distributed Collectives 复习文档"
    section 3): every input travels once around the ring and each device adds
    what arrives, x_{d-1} first and its own x_d last, into an accumulator
    that starts at zero.  fp32 and int32.  Returns (acc, slots) after `steps`
    steps (default P): acc (P, n), slots (P, 2, n) -- the two receive slots
    of every device (the page's hbm_buf[0], hbm_buf[1]; 0 where never
    written)."""
    x = np.ascontiguousarray(x)
    P, n = x.shape
    steps = P if steps is None else steps
    acc = np.empty_like(x)
    slots = np.empty((P, 2, n), dtype=x.dtype)
    lib = _load()
    if x.dtype == np.float32:
        rc = lib.oracle_psum_circ_f32(_ptr(x), _ptr(acc), _ptr(slots), P, n, steps)
    elif x.dtype == np.int32:
        rc = lib.oracle_psum_circ_i32(_ptr(x), _ptr(acc), _ptr(slots), P, n, steps)
    else:
        raise TypeError("psum_circulating: fp32 or int32 (bf16: psum_circulating_bf16)")
    _check(rc, "psum_circulating")
    return acc, slots


def psum_circulating_bf16(x: np.ndarray) -> np.ndarray:
    """bf16 circulating psum: fp32 accumulator, one rounding per device."""
    x = _ranks(x, np.uint16)
    P, n = x.shape
    dst = np.empty_like(x)
    _check(_load().oracle_psum_circ_bf16(_ptr(x), _ptr(dst), P, n), "psum_circulating_bf16")
    return dst


def all_gather(state: np.ndarray, rounds: int | None = None) -> np.ndarray:
    """Ring all-gather applied to `state` (chunk r of row r is rank r's piece)."""
    out = np.array(state, copy=True, order="C")
    P = out.shape[0]
    rounds = P - 1 if rounds is None else rounds
    _check(_load().oracle_all_gather(_ptr(out), P, out[0].size, out.itemsize, rounds),
           "all_gather")
    return out


def all_gather_pieces(pieces: np.ndarray, fill=0) -> np.ndarray:
    """All-gather from compact pieces (P, C): returns (P, P*C)."""
    pieces = np.ascontiguousarray(pieces)
    P = pieces.shape[0]
    C = pieces[0].size
    state = np.full((P, P * C), fill, dtype=pieces.dtype)
    _check(_load().oracle_all_gather_place(_ptr(pieces), _ptr(state), P, P * C,
                                           pieces.itemsize), "all_gather_place")
    return all_gather(state)


def all_reduce(x: np.ndarray) -> np.ndarray:
    """Ring all-reduce: reduce-scatter then all-gather (fp32 / int32)."""
    x = np.ascontiguousarray(x)
    P = x.shape[0]
    out = np.empty_like(x)
    lib = _load()
    if x.dtype == np.float32:
        rc = lib.oracle_all_reduce_f32(_ptr(x), _ptr(out), P, x[0].size)
    elif x.dtype == np.int32:
        rc = lib.oracle_all_reduce_i32(_ptr(x), _ptr(out), P, x[0].size)
    else:
        raise TypeError("all_reduce: fp32 or int32 (bf16: all_reduce_bf16)")
    _check(rc, "all_reduce")
    return out


# --------------------------------------------------------------------------
# bf16 (stored as uint16 bit patterns)
# --------------------------------------------------------------------------
def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) -> uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_bf16_from_f32_array(_ptr(x), _ptr(y), x.size)
    return y


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def reduce_scatter_bf16(x: np.ndarray, rounds: int | None = None):
    """bf16 ring reduce-scatter with an fp32 carry; returns (dst, carry)."""
    x = _ranks(x, np.uint16)
    P = x.shape[0]
    rounds = P - 1 if rounds is None else rounds
    dst = np.empty_like(x)
    carry = np.empty(x.shape, dtype=np.float32)
    _check(_load().oracle_reduce_scatter_bf16(_ptr(x), _ptr(dst), _ptr(carry), P,
                                              x[0].size, rounds), "reduce_scatter_bf16")
    return dst, carry


def reduce_scatter_bidir_bf16(x: np.ndarray, steps: int | None = None):
    """bf16 bidirectional reduce-scatter with fp32 partial sums and one
    rounding of the complete block; returns (dst, carry)."""
    x = _ranks(x, np.uint16)
    P = x.shape[0]
    steps = P if steps is None else steps
    dst = np.empty_like(x)
    carry = np.empty(x.shape, dtype=np.float32)
    _check(_load().oracle_reduce_scatter_bidir_bf16(_ptr(x), _ptr(dst), _ptr(carry), P,
                                                    x[0].size, steps), "reduce_scatter_bidir_bf16")
    return dst, carry


def all_reduce_bf16(x: np.ndarray) -> np.ndarray:
    """bf16 ring all-reduce: fp32 carry, one rounding at the owner, bf16 gather."""
    x = _ranks(x, np.uint16)
    P = x.shape[0]
    dst = np.empty_like(x)
    carry = np.empty(x.shape, dtype=np.float32)
    _check(_load().oracle_all_reduce_bf16(_ptr(x), _ptr(dst), _ptr(carry), P, x[0].size),
           "all_reduce_bf16")
    return dst


# --------------------------------------------------------------------------
# plain references for tolerance checks
# --------------------------------------------------------------------------
def rank_sum_f64(x: np.ndarray, bf16: bool = False):
    """(sum, sum of magnitudes) over ranks in rank order, in fp64."""
    x = np.ascontiguousarray(x)
    P = x.shape[0]
    n = x[0].size
    s = np.empty(n, dtype=np.float64)
    m = np.empty(n, dtype=np.float64)
    lib = _load()
    if bf16:
        rc = lib.oracle_rank_sum_f64_bf16(_ptr(_ranks(x, np.uint16)), P, n, _ptr(s), _ptr(m))
    else:
        rc = lib.oracle_rank_sum_f64_f32(_ptr(_ranks(x, np.float32)), P, n, _ptr(s), _ptr(m))
    _check(rc, "rank_sum_f64")
    return s.reshape(x.shape[1:]), m.reshape(x.shape[1:])


# --------------------------------------------------------------------------
# GEMM + reduce-scatter
# --------------------------------------------------------------------------
def gemm_products_f32(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """C_q = A_q @ B_q for every rank q: bf16 inputs (uint16 bits), fp64
    product, one rounding to fp32.  A: (P, M, K), B: (P, K, N) -> (P, M, N)."""
    A = _ranks(A, np.uint16)
    B = _ranks(B, np.uint16)
    P = A.shape[0]
    out = np.empty((P, A.shape[1], B.shape[2]), dtype=np.float32)
    for q in range(P):
        a = bf16_to_f32(A[q]).astype(np.float64)
        b = bf16_to_f32(B[q]).astype(np.float64)
        out[q] = (a @ b).astype(np.float32)
    return out


def gemm_reduce_scatter(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Rank r's output: rows [r*M/P, (r+1)*M/P) of sum_q A_q B_q, where the
    per-rank products are fp32 and the sum over ranks follows the fp32 ring
    reduce-scatter over row-block chunks ("TPU 与分布式通信原语", collective
    matmul: full local matmul, then the ring reduce-scatter).  Returns
    (P, M/P, N) fp32."""
    Cq = gemm_products_f32(A, B)
    P, M, N = Cq.shape
    if M % P:
        raise ValueError("M must be divisible by P")
    st = reduce_scatter(Cq.reshape(P, M * N))
    rows = M // P
    return np.stack([st[r].reshape(M, N)[r * rows:(r + 1) * rows] for r in range(P)])


def all_gather_gemm(A_shards: np.ndarray, B: np.ndarray):
    """All-gather then matmul ("TPU 与分布式通信原语", collective matmul: the
    all-gather-matmul kernel gathers the row blocks of x around the ring,
    then multiplies by the local weight).  A_shards: (P, M/P, K) bf16 bits,
    rank q's row block of A; B: (P, K, N) bf16 bits.  Returns (A_full, C):
    A_full (P, M, K) is every rank's gathered A -- the ring all-gather of the
    row blocks (chunk c = rows [c M/P, (c+1) M/P)) -- and C (P, M, N) fp32 is
    A_full[q] @ B[q] (fp64 product, one rounding)."""
    A_shards = _ranks(A_shards, np.uint16)
    B = _ranks(B, np.uint16)
    P, Mc, K = A_shards.shape
    full = all_gather_pieces(A_shards.reshape(P, Mc * K)).reshape(P, P * Mc, K)
    return full, gemm_products_f32(full, B)


def all_gather_gemm_rows_f64(A_shards: np.ndarray, B: np.ndarray, q: int, rows) -> tuple:
    """Sampled reference for all_gather_gemm: rows `rows` of A_full @ B[q] in
    fp64 and the magnitude denominator |A_full[rows]| @ |B[q]|, with A_full
    the concatenation of the row blocks."""
    A_shards = _ranks(A_shards, np.uint16)
    P, Mc, K = A_shards.shape
    rows = np.asarray(rows)
    a = bf16_to_f32(A_shards.reshape(P * Mc, K)[rows]).astype(np.float64)
    b = bf16_to_f32(_ranks(B, np.uint16)[q]).astype(np.float64)
    return a @ b, np.abs(a) @ np.abs(b)


def gemm_reduce_scatter_rows_f64(A: np.ndarray, B: np.ndarray, r: int, rows) -> tuple:
    """Sampled reference: for output rank r and local row indices `rows`,
    the fp64 value of sum_q A_q[i,:] @ B_q and the magnitude denominator
    sum_q |A_q[i,:]| @ |B_q| (each exact product is counted once)."""
    A = _ranks(A, np.uint16)
    B = _ranks(B, np.uint16)
    P, M, _ = A.shape
    g = np.asarray(rows) + r * (M // P)
    s = 0.0
    m = 0.0
    for q in range(P):
        a = bf16_to_f32(A[q][g]).astype(np.float64)
        b = bf16_to_f32(B[q]).astype(np.float64)
        s = s + a @ b
        m = m + np.abs(a) @ np.abs(b)
    return s, m

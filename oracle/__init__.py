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


def all_gather_gemm_f64(A_shards: np.ndarray, B: np.ndarray, q: int) -> tuple:
    """Every element of rank q's product: A_full @ B[q] in fp64 and the
    magnitude |A_full| @ |B[q]|, with A_full the concatenation of the row
    blocks.  Returns two (M, N) arrays."""
    A_shards = _ranks(A_shards, np.uint16)
    P, Mc, _ = A_shards.shape
    return all_gather_gemm_rows_f64(A_shards, B, q, np.arange(P * Mc))


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


def gemm_reduce_scatter_f64(A: np.ndarray, B: np.ndarray, r: int) -> tuple:
    """Every element of output rank r: rows [r M/P, (r+1) M/P) of
    sum_q A_q @ B_q in fp64, and the magnitude sum_q |A_q| @ |B_q| of those
    rows (each exact product counted once).  Returns two (M/P, N) arrays."""
    A = _ranks(A, np.uint16)
    P, M, _ = A.shape
    return gemm_reduce_scatter_rows_f64(A, B, r, np.arange(M // P))


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


# --------------------------------------------------------------------------
# tensor-parallel MLP layer
# --------------------------------------------------------------------------
_GELU_C = np.sqrt(2.0 / np.pi)


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
    -- jax.nn.gelu's default, the activation of the tensor-parallel MLP in
    "TPU 与分布式通信原语" (collective matmul) -- in fp64.  It is evaluated
    through the identity 0.5 (1 + tanh(z)) = 1 / (1 + exp(-2z)), which keeps
    full relative accuracy where 1 + tanh(z) would cancel (large negative x)."""
    x = np.asarray(x, dtype=np.float64)
    t = 2.0 * _GELU_C * (x + 0.044715 * x * x * x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-t))


def _bf16_grid(v: np.ndarray, how) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, fp32's exponent range,
    subnormals spaced 2^-133) with `how` (np.rint: nearest, ties to even;
    np.floor / np.ceil: directed).  Returns fp64 values; |v| beyond bf16's
    largest finite value is not expected here."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                       # v = m 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # below 2^-126: the subnormal spacing
    step = np.ldexp(1.0, e - 8)
    return how(v / step) * step


def bf16_from_f64(v: np.ndarray) -> np.ndarray:
    """One rounding of fp64 values to bf16 (nearest, ties to even) -> uint16."""
    r = _bf16_grid(v, np.rint).astype(np.float32)       # exact: 8 significant bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def bf16_nearest(v: np.ndarray) -> np.ndarray:
    """bf16_from_f64 as fp64 values.  Non-decreasing in v, so the roundings
    of every value in [lo, hi] are the bf16 values in
    [bf16_nearest(lo), bf16_nearest(hi)]."""
    return _bf16_grid(v, np.rint)


def _f64(h: np.ndarray) -> np.ndarray:
    return bf16_to_f32(h).astype(np.float64)


def tp_mlp_layer(x_shards: np.ndarray, W1: np.ndarray, W2: np.ndarray):
    """One layer of the tensor-parallel MLP of "TPU 与分布式通信原语"
    (collective matmul): X = gelu(X @ W1) @ W2 with W1 split by columns and W2
    by rows, one device's view being
        out_shard = ReduceScatter(gelu(AllGather(x_shard) @ W1_i) @ W2_i),
    the activation shards being row blocks (tokens) of X.  Steps, in the
    page's order (all bf16 arrays as uint16 bit patterns):
      1. ring all-gather of the row blocks x_shards (P, M/P, D) -> x_full;
      2. local0 = x_full @ W1[q] (fp64 product), rounded to bf16 (the page's
         bf16 matmul output);
      3. local1 = gelu(local0), rounded to bf16 -> h[q] (P, M, F/P);
      4. local2 = h[q] @ W2[q] (fp64 product) rounded to fp32, then the fp32
         ring reduce-scatter of its row blocks, and the owner's sum rounded
         once to bf16 -> out (P, M/P, D).
    Returns (x_full, h, out)."""
    x_shards = _ranks(x_shards, np.uint16)
    W1 = _ranks(W1, np.uint16)
    W2 = _ranks(W2, np.uint16)
    P, Mq, D = x_shards.shape
    full = all_gather_pieces(x_shards.reshape(P, Mq * D)).reshape(P, P * Mq, D)
    h = np.empty((P, P * Mq, W1.shape[2]), dtype=np.uint16)
    for q in range(P):
        local0 = bf16_from_f64(_f64(full[q]) @ _f64(W1[q]))
        h[q] = bf16_from_f64(gelu_tanh(_f64(local0)))
    partial = gemm_products_f32(h, W2)                      # (P, M, D) fp32
    st = reduce_scatter(partial.reshape(P, -1))
    out = np.stack([bf16_from_f32(st[r].reshape(P * Mq, D)[r * Mq:(r + 1) * Mq]) for r in range(P)])
    return full, h, out


def _exact_in_fp32(a: np.ndarray, b: np.ndarray) -> bool:
    """True if every partial sum of every dot product of a @ b is exact in
    fp32 whatever the order: all products are multiples of a common power of
    two g (the coarsest grid both operands sit on) and sum |a b| < 2^24 g."""
    def lsb_exp(v):
        # the exponent of the lowest set bit of every nonzero value (each v is
        # m 2^e with 0.5 <= |m| < 1 and at most 53 significant bits), min over v
        v = v[v != 0]
        if v.size == 0:
            return None
        m, e = np.frexp(v)
        mi = np.abs(m * 2.0 ** 53).astype(np.int64)          # exact: 53-bit integers
        tz = np.zeros(mi.shape, dtype=np.int64)
        for sh in (32, 16, 8, 4, 2, 1):                      # count trailing zero bits
            low = (mi & ((1 << sh) - 1)) == 0
            tz += np.where(low, sh, 0)
            mi = np.where(low, mi >> sh, mi)
        return int((e - 53 + tz).min())
    la, lb = lsb_exp(a), lsb_exp(b)
    if la is None or lb is None:
        return True                                          # a zero operand: every sum is 0
    g = np.ldexp(1.0, la + lb)
    return float((np.abs(a) @ np.abs(b)).max(initial=0.0)) < 2.0 ** 24 * g


_GELU_ARGMIN = -0.7517916     # gelu's only minimum lies in [-0.7518, -0.7517]


def gelu_fp32_error(x: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Absolute error allowed for gelu(x) = g evaluated in fp32 (the kernel
    evaluates x sigmoid(t), t = 2 sqrt(2/pi) (x + 0.044715 x^3), through an
    exponential e = exp(-|t|) <= 1):
      * t: the constants, the cube and the sum (no cancellation: x and
        0.044715 x^3 have the same sign) carry at most 7 roundings, an
        absolute error of 7 u |t|, so e has a relative error of 7 u |t| plus
        2 units of its own (u = 2^-24);
      * x >= 0: gelu = x / (1 + e), and e's relative error reaches the result
        damped by e / (1 + e) (once e is below u it does not reach it at
        all); x < 0: gelu = x e / (1 + e) carries it undamped;
      * 1 + e, the division and the product add a few units more: 8 in all;
      * the bound used is twice that, relative to |g|;
      * near fp32's underflow (x down to about -10.5, where e is subnormal)
        an absolute |x| 2^-147 covers the spacing of fp32's subnormals, 2^-149
        (below -16 the result is 0 in any evaluation; the floor stays 2^-143,
        which rounds to 0 in bf16).
    The exponential's error grows with |t|; the page's form through tanh
    would instead lose all relative accuracy where 1 + tanh cancels (x below
    about -3.5), which is why an implementation evaluates the logistic."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    t = np.abs(2.0 * _GELU_C * (x + 0.044715 * x * x * x))
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(-t)
        damp = np.where(x >= 0, np.where(e > 0, e / (1.0 + e), 0.0), 1.0)
        tw = np.where(damp > 0, t * damp, 0.0)
        rel = 2.0 * (8.0 + 7.0 * tw) * 2.0 ** -24
        rel_part = np.where(g != 0, rel * np.abs(g), 0.0)
    floor = np.ldexp(np.minimum(np.abs(x), 16.0), -147)
    return rel_part + floor


def tp_mlp_bounds(x_shards: np.ndarray, W1: np.ndarray, W2: np.ndarray, r: int, rows):
    """Reference intervals for tp_mlp_layer at the token rows `rows` of rank
    r's output block, for an implementation that accumulates both products in
    fp32 in any order and evaluates gelu in fp32.

    Returns (h_ref, h_lo, h_hi, s, t):
      h_ref (P, R, F/P) bf16 bits: this oracle's h at those rows;
      h_lo, h_hi (P, R, F/P) fp64: the range of every h an fp32
        implementation may produce (the first product within the
        recursive-summation bound D 2^-24 sum|x w|, or exact when the
        operands' grid makes it so, rounded to bf16; gelu of that within
        gelu_fp32_error, rounded to bf16);
      s (R, D) fp64: sum_q h_ref[q] @ W2[q] at those rows;
      t (R, D) fp64: how far an implementation's fp32 out may lie from s:
        sum_q |h - h_ref| @ |W2[q]| over the h intervals plus
        (F/P + P) 2^-24 sum_q max|h| @ |W2[q]|.
    The bf16 output must lie in [bf16_nearest(s - t), bf16_nearest(s + t)]."""
    x_shards = _ranks(x_shards, np.uint16)
    W1 = _ranks(W1, np.uint16)
    W2 = _ranks(W2, np.uint16)
    P, Mq, D = x_shards.shape
    Fr = W1.shape[2]
    g = np.asarray(rows) + r * Mq
    xr = _f64(x_shards.reshape(P * Mq, D)[g])
    h_ref = np.empty((P, len(g), Fr), dtype=np.uint16)
    h_lo = np.empty((P, len(g), Fr))
    h_hi = np.empty((P, len(g), Fr))
    s = 0.0
    t_h = 0.0
    mag = 0.0
    for q in range(P):
        w1 = _f64(W1[q])
        a = xr @ w1
        err = 0.0 if _exact_in_fp32(xr, w1) else D * 2.0 ** -24 * (np.abs(xr) @ np.abs(w1))
        b = _f64(bf16_from_f64(a))
        h_ref[q] = bf16_from_f64(gelu_tanh(b))
        b_lo, b_hi = bf16_nearest(a - err), bf16_nearest(a + err)
        g_lo = np.minimum(gelu_tanh(b_lo), gelu_tanh(b_hi))
        g_lo = np.where((b_lo < _GELU_ARGMIN) & (b_hi > _GELU_ARGMIN), gelu_tanh(_GELU_ARGMIN), g_lo)
        g_hi = np.maximum(gelu_tanh(b_lo), gelu_tanh(b_hi))
        # gelu's evaluation error at the ends of the range (and at gelu's
        # minimum, where g_lo may sit); each end's own bound
        err_lo = np.maximum(gelu_fp32_error(b_lo, g_lo), gelu_fp32_error(b_hi, g_lo))
        err_hi = np.maximum(gelu_fp32_error(b_lo, g_hi), gelu_fp32_error(b_hi, g_hi))
        h_lo[q] = bf16_nearest(g_lo - err_lo)
        h_hi[q] = bf16_nearest(g_hi + err_hi)
        hr = _f64(h_ref[q])
        w2 = np.abs(_f64(W2[q]))
        s = s + hr @ _f64(W2[q])
        t_h = t_h + np.maximum(hr - h_lo[q], h_hi[q] - hr) @ w2
        mag = mag + np.maximum(np.abs(h_lo[q]), np.abs(h_hi[q])) @ w2
    t = t_h + (Fr + P) * 2.0 ** -24 * mag
    return h_ref, h_lo, h_hi, s, t

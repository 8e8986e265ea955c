"""Python entry points of the ring collectives, one per C-ABI call.

Each takes lists of per-rank torch tensors (device memory supplied by torch),
turns them into pointer arrays and calls the library on torch's current HIP
stream.  Nothing here computes: every step runs in the library's kernels.
"""
from __future__ import annotations

from typing import Sequence

import torch

from . import _native as N

_DT = {torch.float32: N.RING_F32, torch.bfloat16: N.RING_BF16, torch.int32: N.RING_I32}


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError("ring collectives take float32, bfloat16 or int32, got %s" % t.dtype)


def _stream(stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    # torch's current stream on the current device, as a raw handle (the
    # same value as torch.cuda.current_stream().cuda_stream, without
    # building a Stream object on every call)
    return torch._C._cuda_getCurrentRawStream(torch.cuda.current_device())


def _ranks(ts: Sequence[torch.Tensor], what: str, numel: int | None = None, dtype=None):
    if len(ts) < 1 or len(ts) > N.MAX_RANKS:
        raise ValueError("%s: 1..%d rank buffers, got %d" % (what, N.MAX_RANKS, len(ts)))
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s: rank buffers must be contiguous device tensors" % what)
        if t.device != ts[0].device:
            raise ValueError("%s: every rank buffer must be on one device" % what)
        if numel is not None and t.numel() != numel:
            raise ValueError("%s: every rank buffer needs %d elements" % (what, numel))
        if dtype is not None and t.dtype != dtype:
            raise TypeError("%s: mixed dtypes" % what)
    return [t.data_ptr() for t in ts]


def _wsarg(ws: torch.Tensor, what: str):
    """(device pointer, size in bytes) of a caller's workspace tensor; a
    host tensor or a strided view is refused here, before the library could
    hand the kernels an address they cannot use."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("%s: the workspace must be a contiguous device tensor" % what)
    return ws.data_ptr(), ws.numel() * ws.element_size()


def workspace_bytes(op: int, P: int, n: int, dtype: torch.dtype = torch.float32) -> int:
    return int(N.lib().ring_workspace_bytes(op, P, n, _DT[dtype]))


def workspace(op: int, P: int, n: int, dtype: torch.dtype, device=None) -> torch.Tensor:
    """A zero-filled workspace of the size the library asks for."""
    nb = workspace_bytes(op, P, n, dtype)
    return torch.zeros(max(nb, 256), dtype=torch.uint8,
                       device=device if device is not None else "cuda")


def _ordered(ws: torch.Tensor, stream) -> torch.Tensor:
    """A workspace just zero-filled on torch's current stream, made ready for
    a call on `stream`: that stream waits for the fill, and the allocator is
    told the block is in use on `stream`, so it is not handed out again
    before the call's kernels there have finished, even if the caller drops
    the returned workspace at once."""
    if stream is not None and stream != torch.cuda.current_stream(ws.device):
        stream.wait_stream(torch.cuda.current_stream(ws.device))
        ws.record_stream(stream)
    return ws


def _ws(ws, op, P, n, dtype, device, stream=None):
    if ws is None:
        ws = _ordered(workspace(op, P, n, dtype, device), stream)
    return ws


def ppermute(src: Sequence[torch.Tensor], dst: Sequence[torch.Tensor], stream=None) -> None:
    """dst[r] <- src[(r - 1 + P) mod P] (right shift)."""
    n = src[0].numel()
    ps = _ranks(src, "ppermute", n, src[0].dtype)
    pd = _ranks(dst, "ppermute", n, src[0].dtype)
    if len(ps) != len(pd):
        raise ValueError("ppermute: src and dst rank counts differ")
    a, ka = N.ptr_array(ps)
    b, kb = N.ptr_array(pd)
    N.check(N.lib().ring_ppermute(a, b, len(ps), n, _dtype(src[0]), _stream(stream)),
            "ring_ppermute")


def _rs_ar(fn, name, op, src, dst, ws, stream):
    n = src[0].numel()
    P = len(src)
    ps = _ranks(src, name, n, src[0].dtype)
    pd = _ranks(dst, name, n, src[0].dtype)
    if len(pd) != P:
        raise ValueError("%s: src and dst rank counts differ" % name)
    ws = _ws(ws, op, P, n, src[0].dtype, src[0].device, stream)
    a, ka = N.ptr_array(ps)
    b, kb = N.ptr_array(pd)
    N.check(fn(a, b, P, n, _dtype(src[0]), *_wsarg(ws, name), _stream(stream)), name)
    return ws


def reduce_scatter(src, dst, ws=None, stream=None):
    """Ring reduce-scatter: chunk r of dst[r] <- sum over ranks of chunk r."""
    return _rs_ar(N.lib().ring_reduce_scatter, "ring_reduce_scatter", N.OP_REDUCE_SCATTER,
                  src, dst, ws, stream)


def reduce_scatter_bidir(src, dst, ws=None, stream=None):
    """Bidirectional ring reduce-scatter (top halves of the chunks travel
    left, bottom halves right): chunk r of dst[r] <- sum over ranks."""
    return _rs_ar(N.lib().ring_reduce_scatter_bidir, "ring_reduce_scatter_bidir",
                  N.OP_REDUCE_SCATTER_BIDIR, src, dst, ws, stream)


def psum_circulating(src, dst, ws=None, stream=None):
    """Circulating-input psum: every input once around the ring; dst[r] <-
    the sum over ranks, added in the order src[r-1], src[r-2], ..., src[r]."""
    return _rs_ar(N.lib().ring_psum_circulating, "ring_psum_circulating", N.OP_PSUM_CIRCULATING,
                  src, dst, ws, stream)


def all_reduce(src, dst, ws=None, stream=None):
    """Ring all-reduce: every dst[r] <- sum over ranks of src."""
    return _rs_ar(N.lib().ring_all_reduce, "ring_all_reduce", N.OP_ALL_REDUCE,
                  src, dst, ws, stream)


def all_reduce_noalloc(src, dst, stream=None) -> None:
    """ring_all_reduce without a workspace argument: the library's static
    device array serves as the workspace, so the call allocates nothing.
    Calls that overlap in time on one device race (one shared array)."""
    n = src[0].numel()
    P = len(src)
    ps = _ranks(src, "ring_all_reduce_noalloc", n, src[0].dtype)
    pd = _ranks(dst, "ring_all_reduce_noalloc", n, src[0].dtype)
    if len(pd) != P:
        raise ValueError("ring_all_reduce_noalloc: src and dst rank counts differ")
    a, ka = N.ptr_array(ps)
    b, kb = N.ptr_array(pd)
    N.check(N.lib().ring_all_reduce_noalloc(a, b, P, n, _dtype(src[0]), _stream(stream)),
            "ring_all_reduce_noalloc")


def all_gather(dst, src=None, ws=None, stream=None):
    """Ring all-gather.  src=None: chunk r of dst[r] already holds rank r's
    piece; otherwise src[r] is rank r's compact piece (numel = n / P)."""
    n = dst[0].numel()
    P = len(dst)
    pd = _ranks(dst, "ring_all_gather", n, dst[0].dtype)
    keep = []
    if src is not None:
        if len(src) != P:
            raise ValueError("ring_all_gather: src and dst rank counts differ")
        ps = _ranks(src, "ring_all_gather", n // P if n % P == 0 else -1, dst[0].dtype)
        a, ka = N.ptr_array(ps)
        keep.append(ka)
    else:
        a = None
    ws = _ws(ws, N.OP_ALL_GATHER, P, n, dst[0].dtype, dst[0].device, stream)
    b, kb = N.ptr_array(pd)
    N.check(N.lib().ring_all_gather(a, b, P, n, _dtype(dst[0]), *_wsarg(ws, "ring_all_gather"),
                                    _stream(stream)), "ring_all_gather")
    return ws


def gemm_reduce_scatter(A, B, out, ws=None, stream=None):
    """out[r] <- rows [r M/P, (r+1) M/P) of sum_q A[q] @ B[q] (bf16 in, fp32 out)."""
    P = len(A)
    M, K = A[0].shape
    K2, Nn = B[0].shape
    if K2 != K or len(B) != P or len(out) != P:
        raise ValueError("gemm_reduce_scatter: shape mismatch")
    pa = _ranks(A, "gemm_reduce_scatter", M * K, torch.bfloat16)
    pb = _ranks(B, "gemm_reduce_scatter", K * Nn, torch.bfloat16)
    po = _ranks(out, "gemm_reduce_scatter", (M // P) * Nn, torch.float32)
    if ws is None:
        nb = int(N.lib().ring_workspace_bytes(N.OP_GEMM_REDUCE_SCATTER, P, M * Nn, N.RING_F32))
        ws = _ordered(torch.zeros(max(nb, 256), dtype=torch.uint8, device=A[0].device), stream)
    a, ka = N.ptr_array(pa)
    b, kb = N.ptr_array(pb)
    o, ko = N.ptr_array(po)
    N.check(N.lib().gemm_reduce_scatter(a, b, o, P, M, Nn, K, *_wsarg(ws, "gemm_reduce_scatter"),
                                        _stream(stream)), "gemm_reduce_scatter")
    return ws


def all_gather_gemm(A_shard, B, A_full, C, ws=None, stream=None):
    """A_full[r] <- the row blocks A_shard[0..P-1] stacked (ring all-gather);
    C[r] <- A_full[r] @ B[r] (bf16 in, fp32 out), overlapped tile by tile."""
    P = len(A_shard)
    Mc, K = A_shard[0].shape
    K2, Nn = B[0].shape
    M = Mc * P
    if K2 != K or len(B) != P or len(A_full) != P or len(C) != P:
        raise ValueError("all_gather_gemm: shape mismatch")
    pa = _ranks(A_shard, "all_gather_gemm", Mc * K, torch.bfloat16)
    pb = _ranks(B, "all_gather_gemm", K * Nn, torch.bfloat16)
    pf = _ranks(A_full, "all_gather_gemm", M * K, torch.bfloat16)
    pc = _ranks(C, "all_gather_gemm", M * Nn, torch.float32)
    if ws is None:
        nb = int(N.lib().ring_workspace_bytes(N.OP_ALL_GATHER_GEMM, P, M * Nn, N.RING_F32))
        ws = _ordered(torch.zeros(max(nb, 256), dtype=torch.uint8, device=A_shard[0].device), stream)
    a, ka = N.ptr_array(pa)
    b, kb = N.ptr_array(pb)
    f, kf = N.ptr_array(pf)
    c, kc = N.ptr_array(pc)
    N.check(N.lib().all_gather_gemm(a, b, f, c, P, M, Nn, K, *_wsarg(ws, "all_gather_gemm"),
                                    _stream(stream)), "all_gather_gemm")
    return ws


def tp_mlp_workspace(P: int, M: int, D: int, F: int, device=None) -> torch.Tensor:
    """A zero-filled workspace for tp_mlp_layer at these shapes."""
    nb = int(N.lib().tp_mlp_workspace_bytes(P, M, D, F))
    return torch.zeros(max(nb, 256), dtype=torch.uint8, device=device if device is not None else "cuda")


def tp_mlp_layer(x_shard, W1, W2, x_full, h, out, ws=None, stream=None):
    """One tensor-parallel MLP layer over P virtual ranks (bf16 everywhere):
    x_full[r] <- the row blocks x_shard[0..P-1] stacked (ring all-gather);
    h[r] <- bf16(gelu(bf16(x_full[r] @ W1[r]))) (tanh gelu);
    out[r] <- bf16(rows [r M/P, (r+1) M/P) of sum_q h[q] @ W2[q]), fp32 sums.
    W1[r] is column block r of W1 (D x F/P), W2[r] row block r of W2
    (F/P x D).  out may be x_shard itself (a layer in place)."""
    P = len(x_shard)
    Mq, D = x_shard[0].shape
    D2, Fr = W1[0].shape
    M, F = Mq * P, Fr * P
    if D2 != D or tuple(W2[0].shape) != (Fr, D) or not (len(W1) == len(W2) == len(x_full) == len(h) ==
                                                          len(out) == P):
        raise ValueError("tp_mlp_layer: shape mismatch")
    bf = torch.bfloat16
    ptrs = [_ranks(x_shard, "tp_mlp_layer", Mq * D, bf), _ranks(W1, "tp_mlp_layer", D * Fr, bf),
            _ranks(W2, "tp_mlp_layer", Fr * D, bf), _ranks(x_full, "tp_mlp_layer", M * D, bf),
            _ranks(h, "tp_mlp_layer", M * Fr, bf), _ranks(out, "tp_mlp_layer", Mq * D, bf)]
    if ws is None:
        ws = _ordered(tp_mlp_workspace(P, M, D, F, device=x_shard[0].device), stream)
    arrs = [N.ptr_array(p_) for p_ in ptrs]
    N.check(N.lib().tp_mlp_layer(*[a_ for a_, _ in arrs], P, M, D, F, *_wsarg(ws, "tp_mlp_layer"),
                                 _stream(stream)), "tp_mlp_layer")
    return ws


def last_error(ws: torch.Tensor, stream=None):
    """(code, info) left in a workspace by the last kernel (synchronises)."""
    import ctypes
    info = ctypes.c_int(0)
    code = N.lib().ring_last_error(*_wsarg(ws, "ring_last_error"), _stream(stream), ctypes.byref(info))
    return int(code), int(info.value)


def workspace_init(ws: torch.Tensor, stream=None) -> None:
    N.check(N.lib().ring_workspace_init(*_wsarg(ws, "ring_workspace_init"), _stream(stream)),
            "ring_workspace_init")

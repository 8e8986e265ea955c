"""Helpers for the GPU tests: move seeded NumPy rank arrays to device tensors
and back, and poison outputs so unwritten elements show up."""
import sys

import numpy as np
import torch


def note(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu-case] %s" % msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, kind: str):
    """(P, n) NumPy array -> list of P device tensors (one allocation each)."""
    out = []
    for r in range(x.shape[0]):
        row = np.ascontiguousarray(x[r]).reshape(-1)
        if kind == "bf16":
            t = torch.from_numpy(row.view(np.int16)).cuda().view(torch.bfloat16)
        else:
            t = torch.from_numpy(row).cuda()
        out.append(t)
    return out


def poison_like(ts, kind: str):
    out = []
    for t in ts:
        if kind == "f32":
            out.append(torch.full_like(t, float("nan")))
        elif kind == "i32":
            out.append(torch.full_like(t, -559038737))          # 0xDEADBEEF
        else:
            out.append(torch.full((t.numel(),), 0x7FC1, dtype=torch.int16,
                                  device=t.device).view(torch.bfloat16))
    return out


def empty_ranks(P, n, kind):
    dt = {"f32": torch.float32, "i32": torch.int32, "bf16": torch.bfloat16}[kind]
    return poison_like([torch.empty(n, dtype=dt, device="cuda") for _ in range(P)], kind)


def to_host(ts, kind: str) -> np.ndarray:
    torch.cuda.synchronize()
    if kind == "bf16":
        return np.stack([t.view(torch.int16).cpu().numpy().view(np.uint16) for t in ts])
    return np.stack([t.cpu().numpy() for t in ts])


def bits(a: np.ndarray) -> np.ndarray:
    """Compare floats by bit pattern (NaN-safe, -0 vs +0 distinct)."""
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def chunk(a_row: np.ndarray, c: int, C: int) -> np.ndarray:
    return a_row[c * C:(c + 1) * C]


def rs_written_chunks(P):
    """(rank, chunk) pairs the reduce-scatter writes: every chunk except
    (r - 1) mod P at rank r."""
    return [(r, c) for r in range(P) for c in range(P) if c != (r - 1) % P]

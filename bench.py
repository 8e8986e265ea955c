"""Benchmark of the ring collectives on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one ring all-reduce (the reduce-scatter rounds and the all-gather
rounds, 2(P-1) rounds in one launch) over P virtual ranks whose buffers all
sit in this GPU's HBM; inputs are resident before the timed region starts.
Prints one JSON line.  Other workloads (--workload) time one call of another
collective of the same path: the bf16 all-reduce, the one-way and the
bidirectional reduce-scatter, ppermute, and the fused GEMM + reduce-scatter.

Default workload (the headline): P = 8 ranks, 64 Mi fp32 per rank (256 MiB
per rank, 2 GiB in all), normal(0, 1), seed 2, out of place.

`value` is algorithmic GB/s: bytes the ring must move (reduce-scatter round:
2 reads + 1 write of a chunk; all-gather round: 1 read + 1 write; at the
widths actually used) divided by the measured time per step.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure

WORKLOADS = {
    "ar_f32_p8_64Mi": dict(op="all_reduce", P=8, n=64 << 20, kind="f32", seed=2, std=1.0),
    "ar_bf16_p16_128Mi": dict(op="all_reduce", P=16, n=128 << 20, kind="bf16", seed=3, std=1e-2),
    "ar_f32_p4_small": dict(op="all_reduce", P=4, n=4096, kind="f32", seed=0, std=None),
    # int32 (8, 128 P) per rank, uniform [-1000, 1000], seed 1: reduce-scatter
    # and all-gather on their own (latency-bound)
    "rs_i32_p8_small": dict(op="reduce_scatter", P=8, n=8 * 128 * 8, kind="i32", seed=1, std=None),
    "ag_i32_p8_small": dict(op="all_gather", P=8, n=8 * 128 * 8, kind="i32", seed=1, std=None),
    # fused GEMM + reduce-scatter: P = 4, A_q, B_q bf16 4096 x 4096, normal(0, 1/64)
    "gemm_rs_p4_4096": dict(op="gemm_rs", P=4, M=4096, N=4096, K=4096, kind="bf16", seed=4,
                            std=1.0 / 64, n=4096 * 4096),
    # circulating-input psum on the headline inputs (moves P times each buffer)
    "psum_circ_f32_p8_64Mi": dict(op="psum_circulating", P=8, n=64 << 20, kind="f32", seed=2,
                                  std=1.0),
    # fused all-gather + GEMM: P = 4, A 4096 x 4096 in row blocks of 1024,
    # B_q bf16 4096 x 4096, normal(0, 1/64)
    "ag_gemm_p4_4096": dict(op="ag_gemm", P=4, M=4096, N=4096, K=4096, kind="bf16", seed=5,
                            std=1.0 / 64, n=4096 * 4096),
    # one tensor-parallel MLP layer: P = 4, x [8192, 1024] in row blocks of
    # 2048 tokens, W1 [1024, 16384] by columns, W2 [16384, 1024] by rows
    "tp_mlp_p4_8192": dict(op="tp_mlp", P=4, M=8192, D=1024, F=16384, kind="bf16", seed=6),
    # the same layer at the chapter's own 256 tokens (64 per rank: the
    # unfused path; latency-bound)
    "tp_mlp_p4_256": dict(op="tp_mlp", P=4, M=256, D=1024, F=16384, kind="bf16", seed=6),
    # a plain copy of known size (2 x 256 MiB read + written): counter calibration
    "ppermute_f32_p2_64Mi": dict(op="ppermute", P=2, n=64 << 20, kind="f32", seed=2, std=1.0),
    # reduce-scatter alone on the headline inputs: one-way ring, and the
    # bidirectional form (top halves of the chunks travel left, bottom right)
    "rs_f32_p8_64Mi": dict(op="reduce_scatter", P=8, n=64 << 20, kind="f32", seed=2, std=1.0),
    "rs_bidir_f32_p8_64Mi": dict(op="reduce_scatter_bidir", P=8, n=64 << 20, kind="f32", seed=2,
                                 std=1.0),
}
DEFAULT = "ar_f32_p8_64Mi"


def moved_bytes(op: str, P: int, n: int, kind: str) -> int:
    """Algorithmic bytes of one call (reads + writes the ring must make)."""
    C = n // P
    if op == "ppermute":
        return 2 * P * n * (2 if kind == "bf16" else 4)
    if op == "psum_circulating":
        # first send (read + write), P slot reads, P-1 forwards, the result
        return 2 * (P + 1) * n * (2 if kind == "bf16" else 4) * P
    if P == 1:
        return 0
    if op == "reduce_scatter_bidir":
        # P-1 steps that add (as the one-way reduce-scatter rounds), then one
        # that moves the complete halves of every rank's own chunk
        if kind == "bf16":
            rs = C * P * sum(2 + (2 if s == 0 else 4) + 4 for s in range(P - 1))
            return rs + C * P * (4 + 2)
        return (P - 1) * 12 * C * P + 8 * C * P
    if kind == "bf16":
        # carry in fp32: round 0 reads two bf16 and writes fp32; middle rounds
        # read bf16 + fp32 and write fp32; the owner's last round writes bf16.
        rs = 0
        for s in range(P - 1):
            rd = 2 + (2 if s == 0 else 4)
            wr = 2 if s == P - 2 else 4
            rs += rd + wr
        rs *= C * P
        ag = (P - 1) * 4 * C * P
    else:
        rs = (P - 1) * 12 * C * P
        ag = (P - 1) * 8 * C * P
    if op == "reduce_scatter":
        return rs
    if op == "all_gather":
        return ag
    return rs + ag


def mlp_layer_cost(P: int, M: int, D: int, F: int) -> dict:
    """Cost model of one tensor-parallel MLP layer ("TPU 与分布式通信原语",
    collective matmul: the all-gather-matmul and the matmul-reduce-scatter of
    one device take the same flops; a device sends P - 1 shards one way)."""
    per = 2 * M * D * (F // P)
    shard = (M // P) * D * 2
    return {"flop_per_matmul_per_rank": per, "flop": 2 * P * per, "shard_bytes": shard,
            "ring_bytes_per_direction": (P - 1) * shard}


KERNEL_SOURCE = {"ring_step_kernel": ("ring_kernels.hip",), "copy_kernel_tab": ("ring_kernels.hip",),
                 "ring_ll_kernel": ("ring_kernels.hip",),
                 "ring_bidir_kernel": ("ring_kernels.hip",), "ring_psum_kernel": ("ring_kernels.hip",),
                 "gemm_rs_kernel": ("gemm_rs.hip", "gemm_core.h"),
                 "ag_gemm_kernel": ("ag_gemm.hip", "gemm_core.h"),
                 "tp_mlp_layer": ("tp_mlp.hip", "ag_gemm.hip", "gemm_rs.hip", "gemm_core.h")}


KERNEL_HEADERS = ("ring_device.h", "ring_internal.h")

# The low-latency rounds' limits (the library's kLlMaxChunkBytes, kLlMaxBytes).
LL_MAX_CHUNK_BYTES = 256 << 10
LL_MAX_WORD_BYTES = 64 << 20


def _ring_kernel(op: str, P: int, n: int, kind: str) -> str:
    """The kernel a ring call of this shape launches, with the current tuning
    and a workspace of ring_workspace_bytes (which holds the low-latency words
    whenever they fit): the one-way collectives of small chunks run
    ring_ll_kernel."""
    from ring_collectives_amd import _native as N
    if op in ("all_reduce", "reduce_scatter", "all_gather") and P > 1 and not N.get_tuning()["stepwise"]:
        chunk = (n // P) * (2 if kind == "bf16" else 4)
        if (chunk <= min(LL_MAX_CHUNK_BYTES, N.get_tuning()["ll_max_chunk_bytes"])
                and 16 * (P - 1) * n <= LL_MAX_WORD_BYTES):
            return "ring_ll_kernel"
    return {"ppermute": "copy_kernel_tab", "reduce_scatter_bidir": "ring_bidir_kernel",
            "psum_circulating": "ring_psum_kernel"}.get(op, "ring_step_kernel")


def _sha_source(kernel: str) -> str:
    """Hash of the kernel's source file and the device headers it includes."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCE[kernel] + KERNEL_HEADERS:
        with open(os.path.join(ROOT, "ring_collectives_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _traffic(workload: str, kernel: str):
    """HBM-side bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "%s_%s_counters.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.strip()
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != _sha_source(kernel):
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _size(nbytes: int) -> str:
    return "%d MiB" % (nbytes >> 20) if nbytes >= 1 << 20 else "%d KiB" % (nbytes >> 10)


def _make_inputs(w):
    import numpy as np
    from ring_collectives_amd import inputs
    if w["op"] == "gemm_rs":
        return inputs.gemm_operands(w["P"], w["M"], w["N"], w["K"], std=w["std"], seed=w["seed"])
    if w["op"] == "ag_gemm":   # rank q's row block of A (M / P rows), and its B_q
        return inputs.gemm_operands(w["P"], w["M"] // w["P"], w["N"], w["K"], std=w["std"],
                                    seed=w["seed"])
    if w["kind"] == "i32":
        return inputs.to_chunk_major(inputs.ring_i32(w["P"], 8, w["n"] // (8 * w["P"])), w["P"])
    if w["kind"] == "f32" and w["std"] is None:
        return inputs.to_chunk_major(inputs.small_f32(w["P"], (8, 512)), w["P"])
    if w["kind"] == "f32":
        return inputs.normal_f32(w["P"], w["n"], seed=w["seed"], std=w["std"])
    if w["kind"] == "bf16":
        return inputs.normal_bf16(w["P"], w["n"], seed=w["seed"], std=w["std"])
    raise ValueError(w)


def _to_dev(x, kind):
    import numpy as np
    import torch
    out = []
    for r in range(x.shape[0]):
        row = x[r]
        if kind == "bf16":
            out.append(torch.from_numpy(row.view(np.int16)).cuda().view(torch.bfloat16))
        else:
            out.append(torch.from_numpy(row).cuda())
    return out


ORACLE_SAMPLE_SECONDS = 10.0   # the oracle runs its sample again until this much time has passed


def _host_cpu() -> dict:
    """The host CPU the oracle runs on: model name and the threads this
    process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    return {"cpu_model": model, "threads_available": threads}


def _slice_threads(C: int, threads: int) -> int:
    """Threads for the multi-thread oracle leg: at most `threads`, and a
    divisor of the chunk length C so every slice is whole."""
    t = max(1, min(threads, 16))
    while t > 1 and C % t:
        t -= 1
    return t


def _oracle_sliced(fn, x, P, T):
    """Run the oracle function `fn` on T sub-problems in parallel threads and
    reassemble the result.  Sub-problem t takes slice t (C / T elements) of
    every chunk of every rank, so its chunk c holds only elements of the
    original chunk c: the ring schedule, and so every fp32 sum's order, is
    the original one, and the result is bit for bit the single call's.  The
    oracle's C routines release the interpreter lock while they run."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    n = x.shape[1]
    C = n // P
    w = C // T
    v = x.reshape(x.shape[0], P, C)
    out = np.empty_like(x)
    ov = out.reshape(x.shape[0], P, C)

    def part(t):
        sub = np.ascontiguousarray(v[:, :, t * w:(t + 1) * w]).reshape(x.shape[0], P * w)
        ov[:, :, t * w:(t + 1) * w] = fn(sub).reshape(x.shape[0], P, w)

    with ThreadPoolExecutor(T) as ex:
        list(ex.map(part, range(T)))
    return out


def _cpu_baseline(w, x):
    """The oracle as it stands, single-threaded, on the same inputs: the
    whole workload, repeated until ORACLE_SAMPLE_SECONDS have passed; the
    rate is that of one pass."""
    import numpy as np
    import oracle
    P, n = x.shape

    def run():
        if w["op"] == "ppermute":
            return oracle.ppermute(x)
        if w["op"] == "reduce_scatter":
            return oracle.reduce_scatter_bf16(x)[0] if w["kind"] == "bf16" else oracle.reduce_scatter(x)
        if w["op"] == "psum_circulating":
            return (oracle.psum_circulating_bf16(x) if w["kind"] == "bf16"
                    else oracle.psum_circulating(x)[0])
        if w["op"] == "all_gather":
            return oracle.all_gather(x)
        if w["op"] == "reduce_scatter_bidir":
            return (oracle.reduce_scatter_bidir_bf16(x)[0] if w["kind"] == "bf16"
                    else oracle.reduce_scatter_bidir(x))
        if w["kind"] == "bf16":
            return oracle.all_reduce_bf16(x)
        return oracle.all_reduce(x)

    t0 = time.perf_counter()
    want = run()
    reps = 1
    while time.perf_counter() - t0 < ORACLE_SAMPLE_SECONDS:
        run()
        reps += 1
    total = time.perf_counter() - t0
    dt = total / reps
    mb = moved_bytes(w["op"], P, n, w["kind"])
    gbs = mb / dt / 1e9
    cpu = {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "seconds": round(total, 3),
           "sample": "the whole workload (%d ranks x %d elements), one thread, %d passes" % (P, n, reps)}
    cpu.update(_host_cpu())
    # The same oracle on every host thread: sub-problems made of one slice of
    # every chunk keep the ring's order, so the result must be the same bits.
    # Only the collectives whose arithmetic is chunk by chunk take part (the
    # bidirectional reduce-scatter splits chunks in halves: a slice would
    # move those halves).
    sliceable = {"all_reduce", "reduce_scatter", "all_gather", "ppermute", "psum_circulating"}
    T = _slice_threads(n // P, cpu["threads_available"])
    if w["op"] in sliceable and T > 1:
        fn = {
            "ppermute": oracle.ppermute,
            "reduce_scatter": (lambda a: oracle.reduce_scatter_bf16(a)[0]) if w["kind"] == "bf16"
            else oracle.reduce_scatter,
            "psum_circulating": oracle.psum_circulating_bf16 if w["kind"] == "bf16"
            else (lambda a: oracle.psum_circulating(a)[0]),
            "all_gather": oracle.all_gather,
            "all_reduce": oracle.all_reduce_bf16 if w["kind"] == "bf16" else oracle.all_reduce,
        }[w["op"]]
        t0 = time.perf_counter()
        got = _oracle_sliced(fn, x, P, T)
        reps_m = 1
        while time.perf_counter() - t0 < ORACLE_SAMPLE_SECONDS:
            _oracle_sliced(fn, x, P, T)
            reps_m += 1
        total_m = time.perf_counter() - t0
        same = bool(np.array_equal(got.view(np.uint8), want.view(np.uint8)))
        cpu["multi_thread"] = {"value": round(mb / (total_m / reps_m) / 1e9, 3), "unit": "GB/s", "cores": T,
                               "seconds": round(total_m, 3), "passes": reps_m,
                               "same_bits_as_one_thread": same,
                               "sample": "the whole workload as %d sub-problems (one slice of every chunk "
                                         "each) on %d threads, the unchanged oracle on each" % (T, T)}
    return want, cpu


def _gemm_main(args, w):
    """Fused GEMM workloads (GEMM + reduce-scatter, all-gather + GEMM):
    TFLOP/s against the bf16 MFMA peak."""
    import numpy as np
    import torch
    from ring_collectives_amd import _native as N
    from ring_collectives_amd import collectives as rc
    P, M, Nn, K = w["P"], w["M"], w["N"], w["K"]
    op = w["op"]
    print("[bench] workload %s: generating inputs" % args.workload, file=sys.stderr, flush=True)
    A, B = _make_inputs(w)
    torch.cuda.set_device(0)
    a = [torch.from_numpy(A[q].view(np.int16)).cuda().view(torch.bfloat16) for q in range(P)]
    b = [torch.from_numpy(B[q].view(np.int16)).cuda().view(torch.bfloat16) for q in range(P)]
    if op == "gemm_rs":
        out = [torch.empty((M // P, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
        ws = rc.workspace(N.OP_GEMM_REDUCE_SCATTER, P, M * Nn, torch.float32)

        def step():
            rc.gemm_reduce_scatter(a, b, out, ws=ws)
        kernel, what = "gemm_rs_kernel", "GEMM + ring reduce-scatter"
    else:
        full = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
        out = [torch.empty((M, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
        ws = rc.workspace(N.OP_ALL_GATHER_GEMM, P, M * Nn, torch.float32)

        def step():
            rc.all_gather_gemm(a, b, full, out, ws=ws)
        kernel, what = "ag_gemm_kernel", "ring all-gather + GEMM"
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    code, info = rc.last_error(ws)
    if code != 0:
        raise SystemExit("%s reported %s (info %#x)" % (what, N.strerror(code), info))
    kern_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    ms_step = (t1 - t0) * 1e3 / args.steps
    avg = sum(kern_ms) / len(kern_ms)
    flop = 2.0 * P * M * Nn * K
    overlap = _overlap(args, a, b, P, M, Nn, K, avg) if op == "gemm_rs" and not args.no_cpu else None
    print("[bench] %d steps: %.4f ms/step (wall), kernel avg %.4f ms min %.4f max %.4f"
          % (args.steps, ms_step, avg, min(kern_ms), max(kern_ms)), file=sys.stderr, flush=True)
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle
        # The oracle as it stands on the whole workload: NumPy's fp64
        # products (BLAS on every host thread) rounded once to fp32, then (for
        # GEMM + reduce-scatter) the fp32 ring reduce-scatter in C.
        print("[bench] cpu_baseline: the oracle on the whole workload", file=sys.stderr, flush=True)
        oracle_fn = ((lambda: oracle.gemm_reduce_scatter(A, B)) if op == "gemm_rs"
                     else (lambda: oracle.all_gather_gemm(A, B)))
        t = time.perf_counter()
        oracle_fn()
        reps = 1
        while time.perf_counter() - t < ORACLE_SAMPLE_SECONDS:
            oracle_fn()
            reps += 1
        total = time.perf_counter() - t
        cpu = {"value": round(flop / (total / reps) / 1e12, 6), "unit": "TFLOP/s",
               "cores": _host_cpu()["threads_available"], "kind": "oracle", "seconds": round(total, 3),
               "sample": "the whole workload (%s, fp64 NumPy BLAS products rounded to fp32%s), %d passes"
                         % (what, ", then the fp32 ring reduce-scatter" if op == "gemm_rs" else "", reps)}
        cpu.update(_host_cpu())
        # Parity on every element: within the fp32 accumulation bound of the
        # fp64 value (full host products, magnitudes included).
        print("[bench] parity: every element against the fp64 products", file=sys.stderr, flush=True)
        worst = 0.0
        if op == "gemm_rs":
            bound = (K + P) * 2.0 ** -24
            for r in range(P):
                ref, mag = oracle.gemm_reduce_scatter_f64(A, B, r)
                worst = max(worst, float((np.abs(out[r].cpu().numpy().astype(np.float64) - ref) / mag).max()))
            same = True
        else:
            bound = K * 2.0 ** -24
            for q in range(P):
                ref, mag = oracle.all_gather_gemm_f64(A, B, q)
                worst = max(worst, float((np.abs(out[q].cpu().numpy().astype(np.float64) - ref) / mag).max()))
            gathered = A.reshape(M, K)
            same = all(np.array_equal(t_.view(torch.int16).cpu().numpy().view(np.uint16), gathered)
                       for t_ in full)
        parity = bool(worst <= bound and same)
        print("[bench] every element: max normalised error %.3e (bound %.3e)%s"
              % (worst, bound, "" if op == "gemm_rs" else ", gathered A exact: %s" % same),
              file=sys.stderr, flush=True)
    line = {
        "metric": "%s TFLOP/s, P=%d virtual ranks, bf16 %dx%dx%d per rank" % (what, P, M, Nn, K),
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 (f32 accumulate)", "data": "synthetic",
        "config": {"workload": args.workload, "P": P, "M": M, "N": Nn, "K": K,
                   "flop_per_step": flop, "parallelism": "P virtual ranks on 1 GPU"},
        "roofline": {"bound": "mfma", "achieved": round(flop / (avg * 1e-3) / 1e12, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flop / (avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": _traffic(args.workload, kernel), "kernel": kernel,
                     "kernel_ms_avg": round(avg, 5)},
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
    }
    if overlap is not None:
        line["overlap"] = overlap
    print(json.dumps(line), flush=True)


def _timed(fn, steps, warmup):
    """Average time of fn over `steps` calls after `warmup`, HIP events on
    the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _overlap(args, a, b, P, M, Nn, K, t_fused):
    """How much of the reduce-scatter the fused kernel hides: the same
    products as P separate GEMMs (the P = 1 path of the same kernel, no
    ring) and the same reduce-scatter on fp32 buffers of the products'
    size (the ring kernel), timed apart; efficiency = (T_gemm + T_rs -
    T_fused) / T_rs."""
    import torch
    from ring_collectives_amd import _native as N
    from ring_collectives_amd import collectives as rc
    C = [torch.empty((M, Nn), dtype=torch.float32, device="cuda") for _ in range(P)]
    ws1 = rc.workspace(N.OP_GEMM_REDUCE_SCATTER, 1, M * Nn, torch.float32)

    def gemms():
        for q in range(P):
            rc.gemm_reduce_scatter([a[q]], [b[q]], [C[q]], ws=ws1)
    t_gemm = _timed(gemms, args.steps, args.warmup)
    src = [c.view(-1) for c in C]
    dst = [torch.empty(M * Nn, dtype=torch.float32, device="cuda") for _ in range(P)]
    ws2 = rc.workspace(N.OP_REDUCE_SCATTER, P, M * Nn, torch.float32)
    t_rs = _timed(lambda: rc.reduce_scatter(src, dst, ws=ws2), args.steps, args.warmup)
    for w_ in (ws1, ws2):
        code, info = rc.last_error(w_)
        if code != 0:
            raise SystemExit("overlap reference reported %s (info %#x)" % (N.strerror(code), info))
    eff = (t_gemm + t_rs - t_fused) / t_rs
    print("[bench] overlap: GEMMs alone %.4f ms, reduce-scatter alone %.4f ms, fused %.4f ms, "
          "efficiency %.2f" % (t_gemm, t_rs, t_fused, eff), file=sys.stderr, flush=True)
    return {"t_gemm_ms": round(t_gemm, 5), "t_rs_ms": round(t_rs, 5), "t_fused_ms": round(t_fused, 5),
            "efficiency": round(eff, 3)}


def _mlp_main(args, w):
    """One tensor-parallel MLP layer (two launches: all-gather + GEMM with the
    gelu epilogue, GEMM + reduce-scatter with the bf16 epilogue): TFLOP/s of
    both products against the bf16 MFMA peak."""
    import numpy as np
    import torch
    from ring_collectives_amd import collectives as rc
    from ring_collectives_amd import inputs
    from ring_collectives_amd import _native as N
    P, M, D, F = w["P"], w["M"], w["D"], w["F"]
    Mq, Fr = M // P, F // P
    print("[bench] workload %s: generating inputs" % args.workload, file=sys.stderr, flush=True)
    x, w1, w2 = inputs.mlp_operands_normal(P, M, D, F, seed=w["seed"])
    torch.cuda.set_device(0)
    dev = lambda a: [torch.from_numpy(a[q].view(np.int16)).cuda().view(torch.bfloat16) for q in range(P)]
    xs, W1, W2 = dev(x), dev(w1), dev(w2)
    bf = torch.bfloat16
    full = [torch.empty((M, D), dtype=bf, device="cuda") for _ in range(P)]
    h = [torch.empty((M, Fr), dtype=bf, device="cuda") for _ in range(P)]
    out = [torch.empty((Mq, D), dtype=bf, device="cuda") for _ in range(P)]
    ws = rc.tp_mlp_workspace(P, M, D, F)

    def step():
        rc.tp_mlp_layer(xs, W1, W2, full, h, out, ws=ws)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    code, info = rc.last_error(ws)
    if code != 0:
        raise SystemExit("tp_mlp_layer reported %s (info %#x)" % (N.strerror(code), info))
    kern_ms = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    ms_step = (t1 - t0) * 1e3 / args.steps
    avg = sum(kern_ms) / len(kern_ms)
    cost = mlp_layer_cost(P, M, D, F)
    flop = cost["flop"]
    print("[bench] %d steps: %.4f ms/step (wall), layer avg %.4f ms min %.4f max %.4f"
          % (args.steps, ms_step, avg, min(kern_ms), max(kern_ms)), file=sys.stderr, flush=True)
    cpu = None
    parity = None
    if not args.no_cpu:
        import oracle
        gf = [t_.view(torch.int16).cpu().numpy().view(np.uint16) for t_ in full]
        gh = np.stack([t_.view(torch.int16).cpu().numpy().view(np.uint16) for t_ in h])
        go = np.stack([t_.view(torch.int16).cpu().numpy().view(np.uint16) for t_ in out])
        # the oracle as it stands on the whole layer (fp64 NumPy BLAS
        # products, gelu in fp64, the fp32 ring reduce-scatter in C)
        print("[bench] cpu_baseline: the oracle on the whole layer", file=sys.stderr, flush=True)
        t = time.perf_counter()
        _, h_ref, out_ref = oracle.tp_mlp_layer(x, w1, w2)
        reps = 1
        while time.perf_counter() - t < ORACLE_SAMPLE_SECONDS:
            oracle.tp_mlp_layer(x, w1, w2)
            reps += 1
        total = time.perf_counter() - t
        cpu = {"value": round(flop / (total / reps) / 1e12, 6), "unit": "TFLOP/s",
               "cores": _host_cpu()["threads_available"], "kind": "oracle", "seconds": round(total, 3),
               "sample": "the whole layer (all-gather, both products in fp64 NumPy BLAS with the bf16 "
                         "roundings and gelu, the fp32 ring reduce-scatter), %d passes" % reps}
        cpu.update(_host_cpu())
        # parity: the gathered input bit for bit; every element's agreement
        # with the oracle's bits (at least 99.9% of h, 98% of the output, as
        # the GPU tests require on plain operands); and 8 sampled tokens per
        # rank inside the oracle's rigorous intervals
        same = all(np.array_equal(g_, x.reshape(M, D)) for g_ in gf)
        h_same = float(np.mean(gh == h_ref))
        o_same = float(np.mean(go == out_ref))
        rows = np.arange(0, Mq, max(Mq // 8, 1))
        ok_h = ok_o = True
        for r in range(P):
            _, lo, hi, s_, t_ = oracle.tp_mlp_bounds(x, w1, w2, r, rows)
            for q in range(P):
                hv = oracle.bf16_to_f32(gh[q][r * Mq + rows]).astype(np.float64)
                ok_h &= bool(np.all((lo[q] <= hv) & (hv <= hi[q])))
            ov = oracle.bf16_to_f32(go[r][rows]).astype(np.float64)
            ok_o &= bool(np.all((oracle.bf16_nearest(s_ - t_) <= ov) & (ov <= oracle.bf16_nearest(s_ + t_))))
        parity = bool(same and ok_h and ok_o and h_same >= 0.999 and o_same >= 0.98)
        print("[bench] gathered x exact: %s; h equal to the oracle's %.5f, out %.5f; sampled h in bounds: %s, "
              "sampled out in bounds: %s" % (same, h_same, o_same, ok_h, ok_o), file=sys.stderr, flush=True)
    line = {
        "metric": "tensor-parallel MLP layer TFLOP/s, P=%d virtual ranks, bf16 x[%d,%d] W1[%d,%d] W2[%d,%d]"
                  % (P, M, D, D, F, F, D),
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 (f32 accumulate)", "data": "synthetic",
        "config": {"workload": args.workload, "P": P, "tokens": M, "d_model": D, "d_hidden": F,
                   "operands": "plain normal bf16: x N(0,1), W1 N(0,1/D), W2 N(0,1/F)",
                   "flop_per_step": flop, "parallelism": "P virtual ranks on 1 GPU"},
        "roofline": {"bound": "mfma", "achieved": round(flop / (avg * 1e-3) / 1e12, 2),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flop / (avg * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "traffic": _traffic(args.workload, "tp_mlp_layer"),
                     "kernel": ("tp_mlp_layer (ag_gemm_kernel + gemm_rs_kernel)" if M % (256 * P) == 0 else
                                "tp_mlp_layer (unfused: ring all-gather, batched GEMM with gelu, batched "
                                "split-K GEMM, ring reduce-scatter of the range sums with the bf16 result)"),
                     "kernel_ms_avg": round(avg, 5)},
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU reaches its steady clocks only after some 100 ms of work: the
    # fused GEMMs measured 9% slower after 5 warm-up steps than after 200
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the oracle baseline (and the GEMM + RS overlap references)")
    args = ap.parse_args()
    # No garbage collection while timing: a collection inside a step's Python
    # call stalls the launching thread long enough for the GPU to drain its
    # queue, and the stall then counts inside that step's events (seen as one
    # step of 12-16 ms in 250 of the all-gather + GEMM).
    gc.collect()
    gc.disable()
    if args.gpus != 1:
        print("bench.py: this build runs P virtual ranks on ONE GPU; --gpus %d is not "
              "supported (the multi-GPU ring is a design note only)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from ring_collectives_amd import _native as N
    from ring_collectives_amd import collectives as rc

    w = WORKLOADS[args.workload]
    if w["op"] in ("gemm_rs", "ag_gemm"):
        return _gemm_main(args, w)
    if w["op"] == "tp_mlp":
        return _mlp_main(args, w)
    P, n, kind = w["P"], w["n"], w["kind"]
    print("[bench] workload %s: generating inputs" % args.workload, file=sys.stderr, flush=True)
    x = _make_inputs(w)
    torch.cuda.set_device(0)
    src = _to_dev(x, kind)
    dst = [torch.empty_like(t) for t in src]
    op = w["op"]
    ws_op = {"reduce_scatter": N.OP_REDUCE_SCATTER, "reduce_scatter_bidir": N.OP_REDUCE_SCATTER_BIDIR,
             "psum_circulating": N.OP_PSUM_CIRCULATING, "all_gather": N.OP_ALL_GATHER}
    C = n // P
    pieces = [src[r][r * C:(r + 1) * C].clone() for r in range(P)]   # rank r's piece, compact
    ws = rc.workspace(ws_op.get(op, N.OP_ALL_REDUCE), P, n, src[0].dtype)
    stream = torch.cuda.current_stream()
    call = {"ppermute": lambda: rc.ppermute(src, dst),
            "all_reduce": lambda: rc.all_reduce(src, dst, ws=ws),
            "reduce_scatter": lambda: rc.reduce_scatter(src, dst, ws=ws),
            "reduce_scatter_bidir": lambda: rc.reduce_scatter_bidir(src, dst, ws=ws),
            "psum_circulating": lambda: rc.psum_circulating(src, dst, ws=ws),
            "all_gather": lambda: rc.all_gather(dst, src=pieces, ws=ws)}[op]

    def step():
        call()
    kernel = _ring_kernel(op, P, n, kind)

    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    code, info = rc.last_error(ws)
    if code != 0:
        raise SystemExit("ring %s reported %s (info %#x)" % (op, N.strerror(code), info))

    # timed region: K steps, one launch each; events on the launch stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    code, info = rc.last_error(ws)
    if code != 0:
        raise SystemExit("ring %s reported %s (info %#x)" % (op, N.strerror(code), info))
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_step = (t1 - t0) * 1e3 / args.steps
    avg_kern_ms = sum(kern_ms) / len(kern_ms)
    mb = moved_bytes(w["op"], P, n, kind)
    value = mb / (ms_step * 1e-3) / 1e9
    achieved = mb / (avg_kern_ms * 1e-3) / 1e9
    print("[bench] %d steps: %.4f ms/step (wall), kernel avg %.4f ms min %.4f max %.4f"
          % (args.steps, ms_step, avg_kern_ms, min(kern_ms), max(kern_ms)),
          file=sys.stderr, flush=True)

    # The copy ceiling in the same run: the library's ppermute copies every
    # rank's buffer (P n elements read and written) with 16-byte streaming
    # accesses, over the same bytes the workload holds.
    cp = [torch.empty_like(t) for t in src]
    esz = 2 if kind == "bf16" else 4
    copy_ms = _timed(lambda: rc.ppermute(src, cp), max(args.steps, 20), 20)
    copy_gbs = 2.0 * P * n * esz / (copy_ms * 1e-3) / 1e9
    del cp
    print("[bench] copy ceiling: %.4f ms for 2 x %d MiB, %.1f GB/s" % (copy_ms, (P * n * esz) >> 20, copy_gbs),
          file=sys.stderr, flush=True)

    cpu = None
    parity = None
    if not args.no_cpu:
        print("[bench] cpu_baseline: oracle on the same inputs", file=sys.stderr, flush=True)
        want, cpu = _cpu_baseline(w, x)
        if kind == "bf16":
            got = np.stack([t.view(torch.int16).cpu().numpy().view(np.uint16) for t in dst])
        else:
            got = np.stack([t.cpu().numpy() for t in dst]).view(np.uint32)
            want = want.view(np.uint32)
        if op == "reduce_scatter":
            # the one-way reduce-scatter leaves chunk (r - 1) mod P of rank r unwritten
            C = n // P
            for r in range(P):
                c = (r - 1) % P
                got[r, c * C:(c + 1) * C] = want[r, c * C:(c + 1) * C]
        parity = bool(np.array_equal(got, want))
        print("[bench] GPU output bit-exact vs oracle: %s" % parity, file=sys.stderr, flush=True)

    traffic = _traffic(args.workload, kernel)
    line = {
        "metric": "ring %s HBM GB/s & %% of peak, P=%d virtual ranks, %s %s/rank"
                  % (w["op"].replace("_", "-"), P, _size(n * (2 if kind == "bf16" else 4)),
                     {"f32": "fp32", "i32": "int32"}.get(kind, kind)),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16 (f32 accumulate)", "i32": "int32"}[kind],
        "data": "synthetic",
        "config": {"workload": args.workload, "P": P, "elems_per_rank": n,
                   "bytes_per_rank": n * (2 if kind == "bf16" else 4),
                   "moved_bytes_per_step": mb, "parallelism": "P virtual ranks on 1 GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kernel,
                     "kernel_ms_avg": round(avg_kern_ms, 5),
                     "copy_gbs": round(copy_gbs, 2), "frac_vs_copy": round(achieved / copy_gbs, 4),
                     "note": "achieved counts the bytes the ring must move (2 reads + 1 write per "
                             "reduce-scatter element and round, 1 + 1 per all-gather one); a "
                             "neighbour's partial sum written in the previous round is often still in "
                             "the 256 MB Infinity Cache when it is read, so fewer bytes reach DRAM "
                             "than achieved counts, and a plain copy of the same buffers (copy_gbs, "
                             "measured in this run) can be slower than the ring; traffic is "
                             "FETCH_SIZE + WRITE_SIZE, which count Infinity Cache hits too"},
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

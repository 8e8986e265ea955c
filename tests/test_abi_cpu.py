"""Host-side checks of libring_collectives.so that need no GPU: the library
loads, exports every function include/ring_collectives.h declares, sizes
workspaces, and rejects bad arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from ring_collectives_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER_DIR = os.path.join(ROOT, "include")


def _declared_functions():
    names = set()
    for fn in os.listdir(HEADER_DIR):
        if not fn.endswith(".h"):
            continue
        src = open(os.path.join(HEADER_DIR, fn)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        src = re.sub(r"#[^\n]*", " ", src)
        for m in re.finditer(r"\b([A-Za-z_]\w*)\s*\(([^;{}]*)\)\s*;", src):
            names.add(m.group(1))
    return names


def test_library_loads():
    assert N.lib() is not None


def test_every_declared_symbol_is_exported():
    decl = _declared_functions()
    assert {"ring_ppermute", "ring_reduce_scatter", "ring_all_gather", "ring_all_reduce",
            "gemm_reduce_scatter", "ring_reduce_scatter_bidir"} <= decl
    out = subprocess.check_output(["nm", "-D", "--defined-only", N.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = sorted(decl - exported)
    assert not missing, missing
    for name in decl:
        assert hasattr(N.lib(), name)


def test_binding_covers_the_header():
    assert _declared_functions() <= set(N.SIGNATURES)


def test_strerror():
    for code in (N.RING_OK, N.RING_EINVAL, N.RING_EUNSUPPORTED, N.RING_EWORKSPACE,
                 N.RING_EHIP, N.RING_ETIMEOUT, N.RING_EPROTOCOL):
        assert N.strerror(code) != "unknown error"
    assert N.strerror(12345) == "unknown error"


def test_workspace_bytes():
    L = N.lib()
    assert L.ring_workspace_bytes(N.OP_PPERMUTE, 4, 4096, N.RING_F32) == 0
    assert L.ring_workspace_bytes(N.OP_ALL_REDUCE, 0, 4096, N.RING_F32) == 0
    assert L.ring_workspace_bytes(N.OP_ALL_REDUCE, 4, 4097, N.RING_F32) == 0
    assert L.ring_workspace_bytes(N.OP_ALL_REDUCE, 4, 4096, 9) == 0
    f = L.ring_workspace_bytes(N.OP_ALL_REDUCE, 8, 64 << 20, N.RING_F32)
    assert f > 0 and f % 256 == 0
    # bf16 needs an fp32 carry of P * n floats for the reduce-scatter rounds
    b = L.ring_workspace_bytes(N.OP_ALL_REDUCE, 16, 128 << 20, N.RING_BF16)
    assert b >= 16 * (128 << 20) * 4
    ag = L.ring_workspace_bytes(N.OP_ALL_GATHER, 16, 128 << 20, N.RING_BF16)
    assert ag < 16 * (128 << 20) * 4
    # P = 1: a status header and a minimal flag table
    assert L.ring_workspace_bytes(N.OP_ALL_REDUCE, 1, 100, N.RING_I32) >= 256
    # small calls also hold one 8-byte word per element and round, 16 (P - 1) n
    # bytes; chunks over 256 KiB, or more than 8 Mi words, hold none
    for op in (N.OP_ALL_REDUCE, N.OP_REDUCE_SCATTER, N.OP_ALL_GATHER):
        small = L.ring_workspace_bytes(op, 4, 4096, N.RING_F32)
        assert small >= 16 * 3 * 4096
        edge = L.ring_workspace_bytes(op, 4, 4 * (64 << 10), N.RING_F32)      # 256 KiB chunks
        over = L.ring_workspace_bytes(op, 4, 4 * ((64 << 10) + 4), N.RING_F32)
        assert edge >= 16 * 3 * 4 * (64 << 10) > over
    assert L.ring_workspace_bytes(N.OP_ALL_REDUCE, 64, 128 * 1024, N.RING_F32) < 16 * 63 * 128 * 1024


def _fake(ptrs):
    return N.ptr_array(ptrs)


def _call_rs(P, n, dtype=N.RING_F32, src=None, dst=None, ws=0x100000, ws_bytes=1 << 40):
    src = src if src is not None else [0x10000000 + r * 0x1000000 for r in range(P)]
    dst = dst if dst is not None else [0x80000000 + r * 0x1000000 for r in range(P)]
    a, ka = _fake(src)
    b, kb = _fake(dst)
    return N.lib().ring_reduce_scatter(a, b, P, n, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("P", [0, -1, 65])
def test_bad_rank_count(P):
    a, ka = _fake([0x1000] * 70)
    assert N.lib().ring_reduce_scatter(a, a, P, 64, N.RING_F32, 0x100000, 1 << 30, None) == N.RING_EINVAL


def test_bidir_argument_checks():
    L = N.lib()
    a, ka = _fake([0x10000000 + r * 0x1000000 for r in range(4)])
    b, kb = _fake([0x50000000 + r * 0x1000000 for r in range(4)])
    assert L.ring_reduce_scatter_bidir(a, b, 4, 4097, N.RING_F32, 0x100000, 1 << 30, None) == N.RING_EINVAL
    assert L.ring_reduce_scatter_bidir(a, b, 4, 4096, 7, 0x100000, 1 << 30, None) == N.RING_EUNSUPPORTED
    assert L.ring_reduce_scatter_bidir(a, b, 0, 4096, N.RING_F32, 0x100000, 1 << 30, None) == N.RING_EINVAL
    assert L.ring_reduce_scatter_bidir(a, b, 4, 0, N.RING_F32, 0x100000, 1 << 30, None) == N.RING_OK
    # too small a workspace is rejected before any launch
    assert L.ring_reduce_scatter_bidir(a, b, 4, 4096, N.RING_F32, 0x100000, 256, None) == N.RING_EWORKSPACE
    # the bidirectional form tiles each half of a chunk, which can take one
    # tile more than the one-way form (compared where chunks are too large
    # for low-latency words), and never holds those words
    big = 4 * ((64 << 10) + 4)
    w = L.ring_workspace_bytes(N.OP_REDUCE_SCATTER_BIDIR, 4, big, N.RING_F32)
    assert w >= L.ring_workspace_bytes(N.OP_REDUCE_SCATTER, 4, big, N.RING_F32) > 0
    assert 0 < L.ring_workspace_bytes(N.OP_REDUCE_SCATTER_BIDIR, 4, 4096, N.RING_F32) < 16 * 3 * 4096
    assert L.ring_workspace_bytes(N.OP_REDUCE_SCATTER_BIDIR, 4, 4097, N.RING_F32) == 0
    wb = L.ring_workspace_bytes(N.OP_REDUCE_SCATTER_BIDIR, 4, 4096, N.RING_BF16)
    assert wb >= 4 * 4096 * 4     # the fp32 partial sums


def test_indivisible_size():
    assert _call_rs(4, 4097) == N.RING_EINVAL


def test_bad_dtype():
    assert _call_rs(4, 4096, dtype=7) == N.RING_EUNSUPPORTED


def test_null_pointers():
    assert N.lib().ring_reduce_scatter(None, None, 4, 4096, N.RING_F32, 0x100000, 1 << 30, None) == N.RING_EINVAL
    src = [0x10000000, 0, 0x30000000, 0x40000000]
    assert _call_rs(4, 4096, src=src) == N.RING_EINVAL


def test_misaligned_pointer():
    src = [0x10000000, 0x20000002, 0x30000000, 0x40000000]
    assert _call_rs(4, 4096, src=src) == N.RING_EINVAL
    # 2-byte alignment is enough for bf16
    assert _call_rs(4, 0, dtype=N.RING_BF16, src=src) == N.RING_OK


def test_overlap_rejected():
    src = [0x10000000 + r * 0x100000 for r in range(4)]
    dst = [0x10000000 + 0x100000 * (r + 1) for r in range(4)]   # dst[r] == src[r+1]
    assert _call_rs(4, 4096, src=src, dst=dst) == N.RING_EINVAL
    dst = [0x90000000 + r * 0x100 for r in range(4)]            # dst buffers overlap each other
    assert _call_rs(4, 4096, src=src, dst=dst) == N.RING_EINVAL


def test_workspace_checks():
    L = N.lib()
    # chunks of 64 Ki + 4 fp32 are too large for low-latency words, so the
    # size below is the flag table's and one byte less must be refused
    n = 4 * ((64 << 10) + 4)
    need = L.ring_workspace_bytes(N.OP_REDUCE_SCATTER, 4, n, N.RING_F32)
    assert _call_rs(4, n, ws_bytes=need - 1) == N.RING_EWORKSPACE
    assert _call_rs(4, 4096, ws=0) == N.RING_EWORKSPACE
    assert _call_rs(4, 4096, ws=0x100010) == N.RING_EWORKSPACE      # not 256-byte aligned


def test_zero_size_is_noop():
    assert _call_rs(8, 0) == N.RING_OK
    a, ka = _fake([0x10000000 + r * 0x1000000 for r in range(4)])
    b, kb = _fake([0x80000000 + r * 0x1000000 for r in range(4)])
    L = N.lib()
    assert L.ring_ppermute(a, b, 4, 0, N.RING_F32, None) == N.RING_OK
    assert L.ring_all_gather(a, b, 4, 0, N.RING_I32, 0x100000, 1 << 30, None) == N.RING_OK
    assert L.ring_all_gather(None, b, 4, 0, N.RING_I32, 0x100000, 1 << 30, None) == N.RING_OK
    assert L.ring_all_reduce(a, b, 4, 0, N.RING_BF16, 0x100000, 1 << 30, None) == N.RING_OK


def test_zero_size_fused_and_two_way_calls_are_noops():
    """M = 0 or N = 0 for the fused GEMMs and the MLP layer, n = 0 for the
    bidirectional reduce-scatter and the circulating psum: RING_OK with no
    launch (the device pointers here are never touched)."""
    L = N.lib()
    P = 4
    a, ka = _fake([0x10000000 + r * 0x1000000 for r in range(P)])
    b, kb = _fake([0x20000000 + r * 0x1000000 for r in range(P)])
    c, kc = _fake([0x30000000 + r * 0x1000000 for r in range(P)])
    d, kd = _fake([0x40000000 + r * 0x1000000 for r in range(P)])
    e, ke = _fake([0x50000000 + r * 0x1000000 for r in range(P)])
    f, kf = _fake([0x60000000 + r * 0x1000000 for r in range(P)])
    ws, wsb = 0x100000, 1 << 30
    assert L.ring_reduce_scatter_bidir(a, b, P, 0, N.RING_F32, ws, wsb, None) == N.RING_OK
    assert L.ring_psum_circulating(a, b, P, 0, N.RING_BF16, ws, wsb, None) == N.RING_OK
    for M, Nn in ((0, 256), (1024, 0)):
        assert L.gemm_reduce_scatter(a, b, c, P, M, Nn, 64, ws, wsb, None) == N.RING_OK
        assert L.all_gather_gemm(a, b, c, d, P, M, Nn, 64, ws, wsb, None) == N.RING_OK
    for M, D, F in ((0, 256, 512), (1024, 0, 512), (1024, 256, 0)):
        assert L.tp_mlp_layer(a, b, c, d, e, f, P, M, D, F, ws, wsb, None) == N.RING_OK


def test_ppermute_rejects_in_place():
    a, ka = _fake([0x10000000 + r * 0x1000000 for r in range(4)])
    assert N.lib().ring_ppermute(a, a, 4, 64, N.RING_F32, None) == N.RING_EINVAL


def test_all_gather_piece_overlap():
    dst = [0x80000000 + r * 0x1000000 for r in range(4)]
    pieces = [d + 16 for d in dst]
    a, ka = _fake(pieces)
    b, kb = _fake(dst)
    assert N.lib().ring_all_gather(a, b, 4, 4096, N.RING_F32, 0x100000, 1 << 30, None) == N.RING_EINVAL


def test_tuning_roundtrip_and_validation():
    old = N.get_tuning()
    try:
        prev = N.set_tuning(tile_vecs=16, map_mode=2)
        assert prev == old
        assert old["gemm_tile_n"] == 0
        assert old["ll_max_chunk_bytes"] == 256 << 10
        N.set_tuning(ll_max_chunk_bytes=0)
        assert N.get_tuning()["ll_max_chunk_bytes"] == 0
        assert N.get_tuning()["tile_vecs"] == 16
        N.set_tuning(gemm_tile_n=256)
        assert N.get_tuning()["gemm_tile_n"] == 256
        assert old["check_flags"] == 0
        N.set_tuning(check_flags=1)
        assert N.get_tuning()["check_flags"] == 1
        for bad in ({"tile_vecs": 5}, {"waves_per_cu": 1}, {"waves_per_cu": 32}, {"map_mode": 1},
                    {"map_mode": 7},
                    {"timeout_s": 0.0}, {"stepwise": 2}, {"drop_round": -1},
                    {"gemm_tile_n": 32}, {"gemm_tile_n": 192},
                    {"ll_max_chunk_bytes": -1}, {"ll_max_chunk_bytes": (256 << 10) + 1},
                    {"check_flags": 2}, {"check_flags": -1}):
            with pytest.raises(N.RingError):
                N.set_tuning(**bad)
    finally:
        t = N.Tuning(**old)
        assert N.lib().ring_set_tuning(ctypes.byref(t)) == N.RING_OK


def test_noalloc_rejects_bad_arguments_before_the_device():
    """ring_all_reduce_noalloc's argument checks run on the host: a null
    pointer array, a bad rank count or dtype, n not divisible by P."""
    L = N.lib()
    fake = [0x10000 * (i + 1) for i in range(4)]
    a, _ = N.ptr_array(fake)
    b, _ = N.ptr_array([p + 0x100000 for p in fake])
    assert L.ring_all_reduce_noalloc(None, b, 4, 4096, N.RING_F32, None) == N.RING_EINVAL
    assert L.ring_all_reduce_noalloc(a, b, 0, 4096, N.RING_F32, None) == N.RING_EINVAL
    assert L.ring_all_reduce_noalloc(a, b, 4, 4097, N.RING_F32, None) == N.RING_EINVAL
    assert L.ring_all_reduce_noalloc(a, b, 4, 4096, 7, None) == N.RING_EUNSUPPORTED
    assert L.ring_all_reduce_noalloc(a, b, 4, 0, N.RING_F32, None) == N.RING_OK


def test_gemm_shapes_whose_views_exceed_2_gib_are_refused():
    """Every buffer view a GEMM tile uses must span less than 2 GiB: B (K x N
    bf16), a 256-row panel of A, 128 rows of an fp32 output.  Shapes past
    that are refused before the device is touched (fake pointers)."""
    L = N.lib()
    P, M = 2, 512
    A, ka = _fake([0x10000000 + r * 0x1000000 for r in range(P)])
    B, kb = _fake([0x40000000 + r * 0x1000000 for r in range(P)])
    C, kc = _fake([0x70000000 + r * 0x1000000 for r in range(P)])
    F, kf = _fake([0xA0000000 + r * 0x1000000 for r in range(P)])
    for Nn, K in ((1024, 1 << 20), (1 << 22, 64), (128, 1 << 22)):
        assert L.gemm_reduce_scatter(A, B, C, P, M, Nn, K, 0x100000, 1 << 40, None) == N.RING_EUNSUPPORTED
        assert L.all_gather_gemm(A, B, F, C, P, M, Nn, K, 0x100000, 1 << 40, None) == N.RING_EUNSUPPORTED

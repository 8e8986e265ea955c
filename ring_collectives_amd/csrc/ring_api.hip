// ring_api.hip -- the C ABI of libring_collectives.so: argument checking,
// workspace layout and launch configuration for the ring collectives.  The
// semantics of every entry point are stated in include/ring_collectives.h.
#include "ring_internal.h"

#include <hip/hip_runtime.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

namespace ringc {

int elem_bytes(int dtype) {
    switch (dtype) {
        case RING_F32: return 4;
        case kDtF32Bf16Out: return 4;
        case RING_I32: return 4;
        case RING_BF16: return 2;
        default: return 0;
    }
}

// Elements one lane handles per tile vector: 16 bytes of fp32/int32; for
// bf16, 4 elements (8 bytes of input, 16 bytes of fp32 carry), so every
// carry store of a wave covers contiguous memory.
int elems_per_vec(int dtype) { return dtype == RING_BF16 ? 4 : (elem_bytes(dtype) ? 16 / elem_bytes(dtype) : 0); }

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Whether a call's workspace holds low-latency words: chunks of at most
// kLlMaxChunkBytes, and the words of all 2(P-1) rounds (P n of them) within
// kLlMaxBytes.  Fixed by the shape alone, so a workspace sized once serves
// whatever the tuning says at call time.
static bool ll_fits(int P, size_t n, int dtype) {
    if (P < 2 || !elem_bytes(dtype)) return false;
    const size_t C = n / (size_t)P;
    return C * (size_t)elem_bytes(dtype) <= kLlMaxChunkBytes &&
           2 * (size_t)(P - 1) * n * sizeof(unsigned long long) <= kLlMaxBytes;
}

RingWs ring_ws_layout(int P, size_t n, int dtype, bool with_ll, size_t tile_elems) {
    RingWs w;
    const size_t C = n / (size_t)P;
    const size_t tile_min = tile_elems ? tile_elems : (size_t)kWave * kMinTileVecs * elems_per_vec(dtype);
    // + 1: the bidirectional reduce-scatter tiles each half of a chunk
    // separately, which can take one tile more than the whole chunk
    const size_t T = (C + tile_min - 1) / tile_min + 1;
    const size_t rows = P > 1 ? 2 * (size_t)(P - 1) : 1;
    w.flags_off = kStatusBytes;
    w.flags_bytes = align_up(rows * (size_t)P * (T ? T : 1) * kFlagStride * sizeof(int), 256);
    w.ll_off = w.flags_off + w.flags_bytes;
    w.ll_bytes = with_ll && ll_fits(P, n, dtype) ? align_up(rows * n * sizeof(unsigned long long), 256) : 0;
    w.carry_off = w.ll_off + w.ll_bytes;
    w.carry_bytes = dtype == RING_BF16 ? align_up((size_t)P * n * sizeof(float), 256) : 0;
    w.total = w.carry_off + w.carry_bytes;
    return w;
}

// Circulating psum: the whole buffer is tiled (no chunks); flag rows 0..P-1
// say a receive slot holds an item, rows P..2P-1 that a slot is free again.
struct PsumWs {
    size_t flags_off, slots_off, total;
};
static PsumWs psum_ws_layout(int P, size_t n, int dtype) {
    PsumWs w;
    const size_t tile_min = (size_t)kWave * kMinTileVecs * elems_per_vec(dtype);
    const size_t T = (n + tile_min - 1) / tile_min;
    w.flags_off = kStatusBytes;
    w.slots_off = w.flags_off + align_up(2 * (size_t)P * (size_t)P * (T ? T : 1) * kFlagStride * sizeof(int), 256);
    w.total = w.slots_off + align_up(2 * (size_t)P * n * (size_t)elem_bytes(dtype), 256);
    return w;
}

static int env_int(const char* name, int dflt) {
    const char* v = getenv(name);
    return v && *v ? atoi(v) : dflt;
}

static bool tuning_valid(const ring_tuning_t& x) {
    return (x.tile_vecs == 4 || x.tile_vecs == 8 || x.tile_vecs == 16) && x.waves_per_cu >= 4 &&
           x.waves_per_cu <= 16 && (x.map_mode == 0 || x.map_mode == 2) && x.timeout_s > 0 &&
           x.timeout_s < 3600 && (x.stepwise == 0 || x.stepwise == 1) && x.drop_round >= 0 &&
           (x.gemm_tile_n == 0 || x.gemm_tile_n == 64 || x.gemm_tile_n == 128 || x.gemm_tile_n == 256) &&
           x.ll_max_chunk_bytes >= 0 && (size_t)x.ll_max_chunk_bytes <= kLlMaxChunkBytes &&
           (x.check_flags == 0 || x.check_flags == 1);
}

static ring_tuning_t& tuning_ref() {
    static ring_tuning_t t = [] {
        ring_tuning_t d;
        // 16 KiB tiles: half the flags and waits of 8 KiB ones; measured
        // 5.25 against 7.16 ms on the P = 8 fp32 circulating psum, 0.836
        // against 0.882 on the bidirectional reduce-scatter, and equal or
        // better on every other bandwidth workload
        d.tile_vecs = 16;
        d.waves_per_cu = 12;
        d.map_mode = 0;
        d.timeout_s = 5.0;
        d.stepwise = 0;
        d.drop_round = 0;
        d.gemm_tile_n = 0;
        d.ll_max_chunk_bytes = (int)kLlMaxChunkBytes;
        d.check_flags = 0;
        ring_tuning_t x = d;
        x.tile_vecs = env_int("RING_TILE_VECS", d.tile_vecs);
        x.waves_per_cu = env_int("RING_WAVES_PER_CU", d.waves_per_cu);
        x.map_mode = env_int("RING_MAP", d.map_mode);
        const char* to = getenv("RING_TIMEOUT_S");
        if (to && *to) x.timeout_s = atof(to);
        x.stepwise = env_int("RING_STEPWISE", 0);
        x.gemm_tile_n = env_int("RING_GEMM_TILE_N", d.gemm_tile_n);
        x.ll_max_chunk_bytes = env_int("RING_LL_MAX_CHUNK_BYTES", d.ll_max_chunk_bytes);
        x.check_flags = env_int("RING_CHECK_FLAGS", 0);
        return tuning_valid(x) ? x : d;
    }();
    return t;
}

ring_tuning_t tuning() { return tuning_ref(); }

DevInfo dev_info() {
    static DevInfo cache[64];
    static int valid[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!valid[dev]) {
        DevInfo d;
        int v = 0;
        d.cus = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0 ? v : 256;
        v = 0;
        d.wall_khz = hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) == hipSuccess && v > 0 ? v : 100000;
        cache[dev] = d;
        valid[dev] = 1;
    }
    return cache[dev];
}

}  // namespace ringc

using namespace ringc;

// ------------------------------------------------------------------ checks
static int check_common(const void* const* a, int P, size_t n, int dtype, bool chunked) {
    if (P < 1 || P > RING_MAX_RANKS) return RING_EINVAL;
    if (!elem_bytes(dtype)) return RING_EUNSUPPORTED;
    if (chunked && n % (size_t)P) return RING_EINVAL;
    if (!a) return RING_EINVAL;
    const size_t al = (size_t)elem_bytes(dtype);
    for (int r = 0; r < P; ++r)
        if (!a[r] || ((uintptr_t)a[r] % al)) return RING_EINVAL;
    return RING_OK;
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// 0: disjoint, 1: exactly in place (dst[r] == src[r] for all r), -1: bad overlap.
static int overlap_kind(const void* const* src, size_t src_bytes, void* const* dst,
                        size_t dst_bytes, int P, bool allow_in_place) {
    if (!src_bytes || !dst_bytes) return 0;
    bool in_place = allow_in_place;
    for (int r = 0; r < P && in_place; ++r) in_place = (src[r] == dst[r]);
    for (int a = 0; a < P; ++a)
        for (int b = a + 1; b < P; ++b)
            if (overlap(dst[a], dst_bytes, dst[b], dst_bytes)) return -1;
    if (in_place) {
        for (int a = 0; a < P; ++a)
            for (int b = 0; b < P; ++b)
                if (a != b && overlap(src[a], src_bytes, dst[b], dst_bytes)) return -1;
        return 1;
    }
    for (int a = 0; a < P; ++a)
        for (int b = 0; b < P; ++b)
            if (overlap(src[a], src_bytes, dst[b], dst_bytes)) return -1;
    return 0;
}

static hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// The occupancy of a ring kernel, queried once per (dtype, tile width,
// kind) and kept: the query costs host time on every call otherwise, which
// small calls feel.  The library targets one architecture, so the answer
// is the same on every device.
static int cached_blocks_per_cu(int dtype, int tile_vecs, int kind) {
    static std::atomic<int> cache[32][17][4];   // dtype codes < 32, tile_vecs <= 16, 4 kinds
    if (dtype < 0 || dtype >= 32 || tile_vecs < 0 || tile_vecs > 16 || kind < 0 || kind > 3)
        return ring_blocks_per_cu(dtype, tile_vecs, kind);
    std::atomic<int>& c = cache[dtype][tile_vecs][kind];
    int v = c.load(std::memory_order_relaxed);
    if (v <= 0) {
        v = ring_blocks_per_cu(dtype, tile_vecs, kind);
        if (v > 0) c.store(v, std::memory_order_relaxed);
    }
    return v;
}

static WsSpan span_hull(WsSpan a, WsSpan b) {
    if (b.hi <= b.lo) return a;
    if (a.hi <= a.lo) return b;
    return WsSpan{a.lo < b.lo ? a.lo : b.lo, a.hi > b.hi ? a.hi : b.hi};
}

// Launch the chunk-step kernel over global rounds [k_begin, k_end) (the
// bidirectional kernel over its rounds 0 .. P-1 when bidir is set).
// extra: a further span of ws the caller's other launches leave data in.
// scratch: ws is the no-alloc entry point's static array -- its flag table
// is sized for the tile this call uses, and the part the call needs zero
// is cleared (a fill kernel) before the launch.
static int run_ring(const void* const* src, void* const* dst, int P, size_t n, int dtype,
                    void* ws, size_t ws_bytes, void* stream, int k_begin, int k_end,
                    int compact_src, int bidir = 0, void* const* out16 = nullptr,
                    const float* ranges = nullptr, int nranges = 0, WsSpan extra = WsSpan{0, 0},
                    bool scratch = false) {
    // reduce-scatter rounds of bf16 data carry fp32 partial sums
    const bool need_carry = dtype == RING_BF16 && (bidir || k_begin < P - 1);
    auto need = [&](const RingWs& l) { return need_carry ? l.total : l.total - l.carry_bytes; };
    if (!ws || ((uintptr_t)ws & 255)) return RING_EWORKSPACE;
    const ring_tuning_t tu = tuning();
    const DevInfo di = dev_info();
    const int esz = elem_bytes(dtype);
    const long long C = (long long)(n / (size_t)P);
    // The layout follows from the shape and the workspace's size alone: a
    // workspace that holds this shape's low-latency words (the size
    // ring_workspace_bytes gives does; one sized for a larger call may hold
    // only the flags) keeps them, and the bf16 carry after them, whether or
    // not this call runs those rounds.  So a call in the flag rounds never
    // leaves its carry where the same shape's words lie.
    const size_t lay_tile = scratch ? (size_t)kWave * tu.tile_vecs * elems_per_vec(dtype) : 0;
    const RingWs with_ll = ring_ws_layout(P, n, dtype, true, lay_tile);
    const bool has_ll = with_ll.ll_bytes && ws_bytes >= need(with_ll);
    const RingWs lay = has_ll ? with_ll : ring_ws_layout(P, n, dtype, false, lay_tile);
    if (ws_bytes < need(lay)) return RING_EWORKSPACE;
    // Low-latency rounds for small one-way calls where the workspace holds
    // their words (not in stepwise mode, whose rounds are separate launches
    // ordered by the stream).
    const bool ll = has_ll && !bidir && !tu.stepwise && (size_t)C * (size_t)esz <= (size_t)tu.ll_max_chunk_bytes;
    if (nranges > 0 && !ll) return RING_EUNSUPPORTED;   // ranges are summed in those rounds only
    const int tile = ll ? kWave * kLlVec : kWave * tu.tile_vecs * elems_per_vec(dtype);
    const long long h = C - C / 2;   // top half of a chunk (bidirectional)
    const int T_top = bidir ? (int)((h + tile - 1) / tile) : 0;
    const int T = bidir ? T_top + (int)((C - h + tile - 1) / tile) : (int)((C + tile - 1) / tile);

    RingParams prm;
    memset(&prm, 0, sizeof prm);
    int vec_ok = ((C * esz) % 16) == 0 && (!bidir || ((h * esz) % 16) == 0);
    for (int r = 0; r < P; ++r) {
        prm.src[r] = src ? src[r] : nullptr;
        prm.dst[r] = dst[r];
        if ((uintptr_t)dst[r] & 15) vec_ok = 0;
        if (src && ((uintptr_t)src[r] & 15)) vec_ok = 0;
    }
    if (out16) {
        for (int r = 0; r < P; ++r) {
            prm.out16[r] = out16[r];
            if ((uintptr_t)out16[r] & 15) vec_ok = 0;
        }
    }
    prm.carry = need_carry && !ll ? (float*)((char*)ws + lay.carry_off) : nullptr;
    prm.ll = ll ? (unsigned long long*)((char*)ws + lay.ll_off) : nullptr;
    prm.ranges = ranges;
    prm.nranges = nranges;
    prm.flags = (int*)((char*)ws + lay.flags_off);
    prm.status = (Status*)ws;
    prm.n = (long long)n;
    prm.C = C;
    prm.spin_limit = (long long)(tu.timeout_s * (double)di.wall_khz * 1000.0);
    prm.P = P;
    prm.T = T;
    prm.tile = tile;
    prm.k_begin = k_begin;
    prm.k_end = k_end;
    prm.vec_ok = vec_ok;
    prm.compact_src = compact_src;
    prm.bidir = bidir;
    prm.T_top = T_top;
    prm.h = h;
    // the flag rounds need their flags zero, the low-latency rounds their
    // words; the bf16 carry of the flag rounds is data left behind.  The
    // span checked runs from the end of the status block (see ws_add_data).
    prm.ws_zero = WsSpan{kStatusBytes, ll ? lay.ll_off + lay.ll_bytes : lay.flags_off + lay.flags_bytes};
    prm.ws_data = span_hull(prm.carry ? WsSpan{lay.carry_off, lay.carry_off + lay.carry_bytes} : WsSpan{0, 0},
                            extra);
    prm.check_flags = tu.check_flags;

    // Grid: a wave waits only for waves of its own ring (P consecutive waves
    // of the dispatch order), so the launch progresses with part of it
    // resident.  Stay within half the occupancy limit: margin for anything
    // else resident.
    int occ = cached_blocks_per_cu(dtype, tu.tile_vecs, ll ? 3 : bidir);
    if (occ < 1) return RING_EHIP;
    int bpc = (tu.waves_per_cu + kWavesPerBlock - 1) / kWavesPerBlock;
    if (bpc > occ / 2) bpc = occ / 2 > 0 ? occ / 2 : 1;
    const long long max_blocks = (long long)di.cus * bpc;
    const long long max_waves = max_blocks * kWavesPerBlock;
    int map_mode = ll ? 0 : tu.map_mode;
    long long blocks = 0;
    int W = 0;
    if (map_mode == 2) {
        long long m = ((long long)T + 7) / 8;
        const long long cap = max_waves / (8LL * P);
        if (m > cap) m = cap;
        while (m >= 1 && 8 * (((long long)P * m + kWavesPerBlock - 1) / kWavesPerBlock) > max_blocks) --m;
        if (m >= 1) {
            W = (int)(8 * m);
            blocks = 8 * (((long long)P * m + kWavesPerBlock - 1) / kWavesPerBlock);
        } else {
            map_mode = 0;
        }
    }
    if (map_mode != 2) {
        long long w = max_waves / P;
        if (w > T) w = T;
        if (w < 1) return RING_EUNSUPPORTED;   // more ranks than resident waves
        W = (int)w;
        blocks = ((long long)P * W + kWavesPerBlock - 1) / kWavesPerBlock;
    }
    prm.waves_per_rank = W;
    prm.map_mode = map_mode;
    prm.drop_round = tu.drop_round;
    if (scratch && launch_fill_zero(ws, prm.ws_zero.hi, as_stream(stream)) != hipSuccess) return RING_EHIP;
    if (tu.stepwise) {
        // One launch per round: stream order replaces the flags (no waits,
        // no signals inside a launch of a single round).
        for (int k = k_begin; k < k_end; ++k) {
            prm.k_begin = k;
            prm.k_end = k + 1;
            if (launch_ring(prm, dtype, tu.tile_vecs, (int)blocks, as_stream(stream)) != hipSuccess)
                return RING_EHIP;
        }
        return RING_OK;
    }
    if (launch_ring(prm, dtype, tu.tile_vecs, (int)blocks, as_stream(stream)) != hipSuccess)
        return RING_EHIP;
    return RING_OK;
}

// Launch the circulating psum kernel.
static int run_psum(const void* const* src, void* const* dst, int P, size_t n, int dtype, void* ws,
                    size_t ws_bytes, void* stream) {
    const PsumWs lay = psum_ws_layout(P, n, dtype);
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < lay.total) return RING_EWORKSPACE;
    const ring_tuning_t tu = tuning();
    const DevInfo di = dev_info();
    const int esz = elem_bytes(dtype);
    const int tile = kWave * tu.tile_vecs * elems_per_vec(dtype);
    const int T = (int)(((long long)n + tile - 1) / tile);
    RingParams prm;
    memset(&prm, 0, sizeof prm);
    int vec_ok = (((long long)n * esz) % 16) == 0;
    for (int r = 0; r < P; ++r) {
        prm.src[r] = src[r];
        prm.dst[r] = dst[r];
        if (((uintptr_t)src[r] | (uintptr_t)dst[r]) & 15) vec_ok = 0;
    }
    prm.flags = (int*)((char*)ws + lay.flags_off);
    prm.slots = (char*)ws + lay.slots_off;
    prm.status = (Status*)ws;
    prm.n = (long long)n;
    prm.C = (long long)n;
    prm.spin_limit = (long long)(tu.timeout_s * (double)di.wall_khz * 1000.0);
    prm.P = P;
    prm.T = T;
    prm.tile = tile;
    prm.vec_ok = vec_ok;
    prm.psum = 1;
    prm.drop_round = tu.drop_round;
    prm.ws_zero = WsSpan{kStatusBytes, lay.slots_off};
    prm.ws_data = WsSpan{lay.slots_off, lay.total};
    prm.check_flags = tu.check_flags;
    // every wave of a tile position's ring must be resident: as run_ring
    int occ = cached_blocks_per_cu(dtype, tu.tile_vecs, 2);
    if (occ < 1) return RING_EHIP;
    int bpc = (tu.waves_per_cu + kWavesPerBlock - 1) / kWavesPerBlock;
    if (bpc > occ / 2) bpc = occ / 2 > 0 ? occ / 2 : 1;
    const long long max_waves = (long long)di.cus * bpc * kWavesPerBlock;
    long long W = max_waves / P;
    if (W > T) W = T;
    if (W < 1) return RING_EUNSUPPORTED;
    prm.waves_per_rank = (int)W;
    prm.map_mode = 0;
    const long long blocks = ((long long)P * W + kWavesPerBlock - 1) / kWavesPerBlock;
    return launch_ring(prm, dtype, tu.tile_vecs, (int)blocks, as_stream(stream)) == hipSuccess ? RING_OK
                                                                                               : RING_EHIP;
}

// ------------------------------------------------------------------ C ABI
int ringc::ring_reduce_scatter_bf16_out(const void* const* src, void* const* dst, void* const* out16, int P,
                                        size_t n, void* ws, size_t ws_bytes, void* stream, WsSpan extra) {
    if (P < 2 || P > RING_MAX_RANKS || !src || !dst || !out16) return RING_EINVAL;
    if (n == 0) return RING_OK;
    if (n % (size_t)P) return RING_EINVAL;
    for (int q = 0; q < P; ++q)
        if (!src[q] || !dst[q] || !out16[q]) return RING_EINVAL;
    return run_ring(src, dst, P, n, kDtF32Bf16Out, ws, ws_bytes, stream, 0, P - 1, 0, 0, out16, nullptr, 0, extra);
}

int ringc::ring_reduce_scatter_ranges_bf16_out(const float* ranges, int S, void* const* out16, int P, size_t n,
                                               void* ws, size_t ws_bytes, void* stream, WsSpan extra) {
    if (P < 2 || P > RING_MAX_RANKS || !ranges || !out16 || S < 1 || S > kLlMaxRanges) return RING_EINVAL;
    if (n == 0) return RING_OK;
    if (n % (size_t)P || ((uintptr_t)ranges & 3)) return RING_EINVAL;
    void* dst[RING_MAX_RANKS];   // the kernel takes dst views; nothing is stored there
    for (int q = 0; q < P; ++q) {
        if (!out16[q]) return RING_EINVAL;
        dst[q] = (void*)(ranges + (size_t)q * n);
    }
    return run_ring(nullptr, dst, P, n, kDtF32Bf16Out, ws, ws_bytes, stream, 0, P - 1, 0, 0, out16, ranges, S,
                    extra);
}

extern "C" {

size_t ring_workspace_bytes(int op, int P, size_t n, int dtype) {
    if (P < 1 || P > RING_MAX_RANKS) return 0;
    switch (op) {
        case RING_OP_PPERMUTE: return 0;
        case RING_OP_REDUCE_SCATTER:
        case RING_OP_ALL_REDUCE:
            if (!elem_bytes(dtype) || n % (size_t)P) return 0;
            return ring_ws_layout(P, n, dtype).total;
        case RING_OP_REDUCE_SCATTER_BIDIR:   // never in the low-latency rounds
            if (!elem_bytes(dtype) || n % (size_t)P) return 0;
            return ring_ws_layout(P, n, dtype, false).total;
        case RING_OP_ALL_GATHER: {
            if (!elem_bytes(dtype) || n % (size_t)P) return 0;
            RingWs w = ring_ws_layout(P, n, dtype);
            return w.total - w.carry_bytes;   // a copy needs no carry
        }
        case RING_OP_GEMM_REDUCE_SCATTER:
            return gemm_rs_workspace_bytes(P, n);
        case RING_OP_ALL_GATHER_GEMM:
            return ag_gemm_workspace_bytes(P, n);
        case RING_OP_PSUM_CIRCULATING:
            if (!elem_bytes(dtype)) return 0;
            return psum_ws_layout(P, n, dtype).total;
        default: return 0;
    }
}

int ring_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws) return RING_EINVAL;
    if (!ws_bytes) return RING_OK;
    return launch_fill_zero(ws, ws_bytes, as_stream(stream)) == hipSuccess ? RING_OK : RING_EHIP;
}

int ring_ppermute(const void* const* src, void* const* dst, int P, size_t n, int dtype,
                  void* stream) {
    // a whole-buffer shift: no chunking, so P need not divide n
    int rc = check_common(src, P, n, dtype, false);
    if (rc) return rc;
    if ((rc = check_common(dst, P, n, dtype, false))) return rc;
    const size_t bytes = n * (size_t)elem_bytes(dtype);
    if (overlap_kind(src, bytes, dst, bytes, P, false) != 0) return RING_EINVAL;
    if (n == 0) return RING_OK;
    return launch_copy(src, dst, P, bytes, 1, as_stream(stream)) == hipSuccess ? RING_OK : RING_EHIP;
}

enum { KIND_RS, KIND_AR, KIND_RS_BIDIR };

static int rs_or_ar(const void* const* src, void* const* dst, int P, size_t n, int dtype,
                    void* ws, size_t ws_bytes, void* stream, int kind, bool scratch = false) {
    int rc = check_common(src, P, n, dtype, true);
    if (rc) return rc;
    if ((rc = check_common(dst, P, n, dtype, true))) return rc;
    const size_t bytes = n * (size_t)elem_bytes(dtype);
    const int ov = overlap_kind(src, bytes, dst, bytes, P, true);
    if (ov < 0) return RING_EINVAL;
    if (n == 0) return RING_OK;
    if (P == 1) {   // no rounds: the sum over one rank is its input
        if (ov == 1) return RING_OK;
        return launch_copy(src, dst, 1, bytes, 0, as_stream(stream)) == hipSuccess ? RING_OK : RING_EHIP;
    }
    if (kind == KIND_RS_BIDIR)   // P steps: P-1 that add, one that takes the complete halves
        return run_ring(src, dst, P, n, dtype, ws, ws_bytes, stream, 0, P, 0, 1);
    if (scratch && !ws) return RING_EHIP;   // the static array's address was not available
    return run_ring(src, dst, P, n, dtype, ws, ws_bytes, stream, 0,
                    kind == KIND_AR ? 2 * (P - 1) : P - 1, 0, 0, nullptr, nullptr, 0, WsSpan{0, 0}, scratch);
}

int ring_reduce_scatter(const void* const* src, void* const* dst, int P, size_t n, int dtype,
                        void* ws, size_t ws_bytes, void* stream) {
    return rs_or_ar(src, dst, P, n, dtype, ws, ws_bytes, stream, KIND_RS);
}

int ring_reduce_scatter_bidir(const void* const* src, void* const* dst, int P, size_t n, int dtype,
                              void* ws, size_t ws_bytes, void* stream) {
    return rs_or_ar(src, dst, P, n, dtype, ws, ws_bytes, stream, KIND_RS_BIDIR);
}

int ring_all_reduce(const void* const* src, void* const* dst, int P, size_t n, int dtype,
                    void* ws, size_t ws_bytes, void* stream) {
    return rs_or_ar(src, dst, P, n, dtype, ws, ws_bytes, stream, KIND_AR);
}

int ring_psum_circulating(const void* const* src, void* const* dst, int P, size_t n, int dtype,
                          void* ws, size_t ws_bytes, void* stream) {
    int rc = check_common(src, P, n, dtype, false);
    if (rc) return rc;
    if ((rc = check_common(dst, P, n, dtype, false))) return rc;
    const size_t bytes = n * (size_t)elem_bytes(dtype);
    if (overlap_kind(src, bytes, dst, bytes, P, true) < 0) return RING_EINVAL;
    if (n == 0) return RING_OK;
    return run_psum(src, dst, P, n, dtype, ws, ws_bytes, stream);
}

}  // extern "C"

int ringc::ring_all_gather_rec(const void* const* src_or_null, void* const* dst, int P, size_t n, int dtype,
                               void* ws, size_t ws_bytes, void* stream, WsSpan extra) {
    int rc = check_common(dst, P, n, dtype, true);
    if (rc) return rc;
    const size_t esz = (size_t)elem_bytes(dtype);
    const size_t bytes = n * esz;
    if (src_or_null) {
        if ((rc = check_common(src_or_null, P, n, dtype, true))) return rc;
        if (overlap_kind(src_or_null, (n / (size_t)P) * esz, dst, bytes, P, false) != 0)
            return RING_EINVAL;
    } else if (overlap_kind(dst, 0, dst, bytes, P, false) < 0) {
        return RING_EINVAL;
    }
    if (n == 0) return RING_OK;
    if (P == 1) {
        if (!src_or_null) return RING_OK;
        return launch_copy(src_or_null, dst, 1, bytes, 0, as_stream(stream)) == hipSuccess ? RING_OK : RING_EHIP;
    }
    // the all-gather rounds are global rounds P-1 .. 2P-3 of the all-reduce
    return run_ring(src_or_null, dst, P, n, dtype, ws, ws_bytes, stream, P - 1, 2 * (P - 1),
                    src_or_null ? 1 : 0, 0, nullptr, nullptr, 0, extra);
}

extern "C" {

int ring_all_gather(const void* const* src_or_null, void* const* dst, int P, size_t n, int dtype,
                    void* ws, size_t ws_bytes, void* stream) {
    return ring_all_gather_rec(src_or_null, dst, P, n, dtype, ws, ws_bytes, stream, WsSpan{0, 0});
}

}  // extern "C"

// ------------------------------------------------------------------ no-alloc entry point
// The static array behind ring_all_reduce_noalloc.  In host code `scratch`
// names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns for the current device may reach a kernel or
// a fill.
static __device__ __align__(256) unsigned char scratch[RING_NOALLOC_SCRATCH_BYTES];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; null if the lookup fails.
static void* scratch_ptr() {
    static std::atomic<void*> ptrs[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = ptrs[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptrs[dev].store(p, std::memory_order_release);
    }
    return p;
}

extern "C" {

int ring_all_reduce_noalloc(const void* const* src, void* const* dst, int P, size_t n, int dtype, void* stream) {
    int rc = check_common(src, P, n, dtype, true);
    if (rc) return rc;
    if ((rc = check_common(dst, P, n, dtype, true))) return rc;
    const size_t bytes = n * (size_t)elem_bytes(dtype);
    if (overlap_kind(src, bytes, dst, bytes, P, true) < 0) return RING_EINVAL;
    if (n == 0) return RING_OK;
    // P = 1 is a copy and needs no scratch; rs_or_ar takes that path first
    return rs_or_ar(src, dst, P, n, dtype, P > 1 ? scratch_ptr() : nullptr, RING_NOALLOC_SCRATCH_BYTES, stream,
                    KIND_AR, true);
}

int ring_last_error(const void* ws, size_t ws_bytes, void* stream, int* info) {
    if (!ws || ws_bytes < kStatusBytes) return RING_EINVAL;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return RING_EHIP;
    Status st;
    if (hipMemcpy(&st, ws, sizeof st, hipMemcpyDeviceToHost) != hipSuccess) return RING_EHIP;
    if (info) *info = st.info;
    return st.code;
}

void ring_get_tuning(ring_tuning_t* t) {
    if (t) *t = tuning_ref();
}

int ring_set_tuning(const ring_tuning_t* t) {
    if (!t || !tuning_valid(*t)) return RING_EINVAL;
    tuning_ref() = *t;
    return RING_OK;
}

const char* ring_strerror(int code) {
    switch (code) {
        case RING_OK: return "ok";
        case RING_EINVAL: return "invalid argument (rank count, size, pointer, alignment or overlap)";
        case RING_EUNSUPPORTED: return "unsupported dtype or shape";
        case RING_EWORKSPACE:
            return "workspace missing, misaligned or too small, or its flags lie over data an earlier call "
                   "left there (re-initialise it)";
        case RING_EHIP: return "HIP runtime call failed";
        case RING_ETIMEOUT: return "a rank waited for its neighbour past the watchdog limit";
        case RING_EPROTOCOL: return "a flag was set twice or a word overwritten before it was read (check_flags)";
        default: return "unknown error";
    }
}

}  // extern "C"

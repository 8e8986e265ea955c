// ring_kernels.hip -- gfx950 kernels of the ring collectives.
//
//   * copy_kernel_tab   : ppermute (dst[r] = src[(r - shift) mod P]), and the
//                         plain copies of the P = 1 cases.
//   * ring_step_kernel  : the persistent chunk-step kernel that runs the ring
//                         reduce-scatter and all-gather rounds for every
//                         virtual rank at once.
//   * ring_bidir_kernel : the bidirectional reduce-scatter (halves of every
//                         chunk travel both ways round the ring).
//   * ring_psum_kernel  : the circulating-input psum (every input once round
//                         the ring, double receive slots, capacity flags).
//   * ring_ll_kernel    : the one-way rounds for small calls, each value
//                         passed on with its own ready mark.
//   * fill_zero_kernel  : workspace initialisation.
//
// Ring schedule ("全归约 3：Ring——每步大小恒定", Walkthrough).  P ranks, chunk
// size C = n / P, left(r) = (r - 1 + P) mod P.  Global round k = 0 .. 2P-3:
//   k <  P-1 : reduce-scatter round s = k, chunk c = (r - s - 2) mod P;
//              dst[r][c] = src[r][c] + (s == 0 ? src[left][c] : dst[left][c])
//   k >= P-1 : all-gather round t = k - (P-1), chunk c = (r - t - 1) mod P;
//              dst[r][c] = dst[left][c]
// Round k of rank r reads what rank left(r) wrote in round k-1 (nothing at the
// first round of a launch: its inputs were complete before the launch).
//
// Synchronisation (same page: one signal row per round, waits "Ge 1", notify
// by atomic add; "Triton-distributed 语义", producer/consumer and
// consume_token sections: store, then signal; wait, then load).  The unit of
// work is a tile: `tile` consecutive elements of one chunk, handled by one
// wavefront.  Flag (k, r, j) in HBM says "rank r has finished tile j of its
// round k-1".  Ranks on different XCDs do not share an L2, so every access
// that crosses ranks carries device scope on the instruction itself: the
// producer's stores are written through to the device coherence point and
// the consumer's loads of its neighbour's data bypass stale L1/L2 copies.
// The producer waits for all its memory operations to complete, then adds 1
// to the flag; the consumer polls the flag until it is >= 1 and only then
// issues the loads of its neighbour's data.  This is the ordering an
// agent-scope release/acquire pair gives, without the whole-L2 write-back and
// invalidate those fences cost per tile.  Each flag is set by one wave and
// read by one wave per launch, so the reader clears it after use and a
// finished launch leaves the table zeroed for the next one.
//
// Work assignment.  Each rank gets `waves_per_rank` waves; wave w of rank r
// takes tile positions j = w, w + W, w + 2W, ... and for each position runs
// every round k in order.  A wave only ever waits for (k-1, left, j), which
// belongs to the left rank's wave with the same w and an earlier place in
// that wave's own order (same j, smaller k).  The P waves sharing a w form a
// closed ring and are placed in consecutive workgroups (or on one XCD), so
// the rings that are resident can always finish and free room for the rest;
// the host also keeps the grid within half the occupancy limit, so normally
// every wave is resident from the start.  A watchdog bounds every wait.
#include "ring_device.h"

#include <hip/hip_runtime.h>

namespace ringc {

enum { DT_F32 = RING_F32, DT_BF16 = RING_BF16, DT_I32 = RING_I32, DT_F32B = kDtF32Bf16Out };

__device__ __forceinline__ int left_of(int r, int P) { return (r - 1 + P) % P; }
__device__ __forceinline__ int rs_chunk(int r, int s, int P) { return (r - s - 2 + 2 * P) % P; }
__device__ __forceinline__ int ag_chunk(int r, int t, int P) { return (r - t - 1 + P) % P; }

// ---------------------------------------------------------------- cache policies
// What each access of the ring kernels is to the caches (chosen by measuring
// the bandwidth workloads with every combination, all bit-identical):
//   OWN  a rank's own input, read once per launch: streamed (NT);
//   RCV  a neighbour's partial sum or chunk: device scope (required, see
//        above) and streamed -- with the bf16 carry, which no cache holds,
//        this alone took the P = 16 all-reduce from 5.1 to 4.3 ms;
//   PUB  what a neighbour reads in a later round: device scope only, so the
//        line can stay in the Infinity Cache for that read (streaming these
//        stores cost the fp32 all-reduce 20%);
//   FIN  results nobody reads in this launch: streamed.
constexpr int POL_OWN = POL_NT;
constexpr int POL_RCV = POL_DEV | POL_NT;
constexpr int POL_PUB = POL_DEV;
constexpr int POL_FIN = POL_NT;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ unsigned bf16_rne(float f) {
    unsigned u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// ---------------------------------------------------------------- flags
__device__ __forceinline__ int* flag_at(const RingParams& p, int k, int r, int j) {
    return p.flags + ((size_t)(k * p.P + r) * p.T + j) * kFlagStride;
}

// Wait for flag (k, left, j): the left neighbour finished tile j of round k-1.
__device__ __forceinline__ int peek_flag(const RingParams& p, int k, int left, int j) {
    return peek_flag(flag_at(p, k, left, j));
}
__device__ __forceinline__ bool wait_flag(const RingParams& p, int k, int left, int r, int j,
                                          int lane, int seen) {
    return wait_flag(flag_at(p, k, left, j), p.status, p.spin_limit, r, k, j, lane, seen);
}
// Set flag (k, r, j): this rank finished tile j of round k-1.
__device__ __forceinline__ void signal_flag(const RingParams& p, int k, int r, int j, int lane) {
    signal_flag(flag_at(p, k, r, j), lane, p.check_flags, p.status, r, k, j);
}

// Start of every ring launch: the first lane of the grid adds the launch's
// data span to the workspace's record, and every wave issues the loads of
// the record it checks (ws_ok) before it first signals a flag or passes a
// word on -- which precedes its first wait, so no wave reads a flag or word
// of a table that holds another call's data.
__device__ __forceinline__ WsRecord ring_launch_begin(const RingParams& p) {
    if (blockIdx.x == 0 && threadIdx.x == 0) ws_add_data(p.status, p.ws_data);
    return ws_record(p.status);
}

// ---------------------------------------------------------------- tile bodies
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { typedef float T; static constexpr int VPE = 4; };
template <> struct Elem<DT_I32> { typedef int T; static constexpr int VPE = 4; };
template <> struct Elem<DT_BF16> { typedef unsigned short T; static constexpr int VPE = 4; };
template <> struct Elem<DT_F32B> { typedef float T; static constexpr int VPE = 4; };

template <int DT> __device__ __forceinline__ unsigned add1(unsigned a, unsigned b);
template <> __device__ __forceinline__ unsigned add1<DT_F32>(unsigned a, unsigned b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
}
template <> __device__ __forceinline__ unsigned add1<DT_I32>(unsigned a, unsigned b) {
    return a + b;   // wraps modulo 2^32
}
template <int DT> __device__ __forceinline__ u32x4 add4(u32x4 a, u32x4 b) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = add1<DT>(a[q], b[q]);
    return o;
}

// Where one tile of round k lives.
struct TilePos {
    long long e0;    // first element of the tile in a rank buffer
    long long off;   // first element of the tile within its chunk
    long long len;   // elements in the tile (the last tile of a chunk may be short)
};
__device__ __forceinline__ TilePos tile_pos(const RingParams& p, int c, int j) {
    TilePos t;
    t.off = (long long)j * p.tile;
    t.e0 = (long long)c * p.C + t.off;
    t.len = (p.C - t.off) < p.tile ? (p.C - t.off) : p.tile;
    return t;
}

// One reduce-scatter round of tile t (position j) of one rank, fp32 / int32:
//   dst[r][t] = src[r][t] + (first ? src[from][t] : dst[from][t])
// after waiting for flag (k, from, j): rank `from` finished the tile.  With
// OUT16 (fp32 only) the owner's round (last) stores the sum rounded once to
// bf16 into out16[r], at the tile's place in the chunk, instead.
template <int DT, int U, bool OUT16 = false>
__device__ bool rs_tile_at(const RingParams& p, int r, int from, int k, int j, const TilePos& t,
                           bool first, int lane, bool wait, bool last = false) {
    constexpr int DA = DT == DT_F32B ? DT_F32 : DT;   // the arithmetic
    const long long nb = t.len * 4;
    const rsrc_t own = tile_view((const char*)p.src[r] + t.e0 * 4, nb);
    const rsrc_t rcv = tile_view((const char*)(first ? p.src[from] : p.dst[from]) + t.e0 * 4, nb);
    const rsrc_t out = tile_view((char*)p.dst[r] + t.e0 * 4, nb);
    const int seen = wait ? peek_flag(p, k, from, j) : 1;
    if (p.vec_ok) {
        u32x4 a[U], b[U];
#pragma unroll
        for (int i = 0; i < U; ++i) a[i] = ld16<POL_OWN>(own, (unsigned)(lane + i * kWave) * 16u);
        if (wait && !wait_flag(p, k, from, r, j, lane, seen)) return false;
#pragma unroll
        for (int i = 0; i < U; ++i) b[i] = ld16<POL_RCV>(rcv, (unsigned)(lane + i * kWave) * 16u);
        if constexpr (OUT16) {
            if (last) {
                const rsrc_t o16 = tile_view((unsigned short*)p.out16[r] + t.off, t.len * 2);
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    const u32x4 x = add4<DA>(a[i], b[i]);
                    u32x2 h;
                    h[0] = pack_bf16(__uint_as_float(x[0]), __uint_as_float(x[1]));
                    h[1] = pack_bf16(__uint_as_float(x[2]), __uint_as_float(x[3]));
                    st8<POL_FIN>(h, o16, (unsigned)(lane + i * kWave) * 8u);
                }
                return true;
            }
        }
#pragma unroll
        for (int i = 0; i < U; ++i) st16<POL_PUB>(add4<DA>(a[i], b[i]), out, (unsigned)(lane + i * kWave) * 16u);
    } else {
        if (wait && !wait_flag(p, k, from, r, j, lane, seen)) return false;
        for (long long i = lane; i < t.len; i += kWave) {
            const unsigned o = (unsigned)i * 4u;
            const unsigned x = add1<DA>(ld4<POL_OWN>(own, o), ld4<POL_RCV>(rcv, o));
            if constexpr (OUT16) {
                if (last) {
                    st2<POL_FIN>((unsigned short)bf16_rne(__uint_as_float(x)),
                                 tile_view((unsigned short*)p.out16[r] + t.off, t.len * 2), (unsigned)i * 2u);
                    continue;
                }
            }
            st4<POL_PUB>(x, out, o);
        }
    }
    return true;
}

// One round of the one-way ring: chunk c = (r - s - 2) mod P from the left.
template <int DT, int U>
__device__ __forceinline__ bool rs_tile(const RingParams& p, int r, int left, int k, int j, int lane,
                                        bool wait) {
    const TilePos t = tile_pos(p, rs_chunk(r, k, p.P), j);
    if constexpr (DT == DT_F32B) return rs_tile_at<DT, U, true>(p, r, left, k, j, t, k == 0, lane, wait, k == p.P - 2);
    else return rs_tile_at<DT, U>(p, r, left, k, j, t, k == 0, lane, wait);
}

// The fp32 carry of a whole bf16 tile (p.tile = 256 U elements) is kept in
// a paired layout: the 8 elements lane l reads as one 16-byte vector i of
// bf16 (elements 8 (64 i + l) .. + 7) have their carry at 16-byte vectors
// 64 (2 i) + l (the first four) and 64 (2 i + 1) + l (the last four) of the
// tile's carry.  Every bf16 access is then 16 bytes per lane and every carry
// access of a wave one contiguous KiB: a round moves 16 bytes per memory
// instruction, as the fp32 rounds do (with 8-byte bf16 accesses it moved 40
// bytes in three instructions, and ran at 6.1 against 7.2 TB/s).  The carry
// never leaves the ring, so only its producer and its consumer see the
// layout; both use it exactly when the tile is whole and vec_ok holds, and
// the short last tile of a chunk keeps the natural order (the paired one
// would put some of its elements beyond the tile).
__device__ __forceinline__ bool carry_paired(const RingParams& p, const TilePos& t) {
    return p.vec_ok && t.len == p.tile;
}
__device__ __forceinline__ void bf16x8_to_f32(const u32x4 v, float (&x)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        x[2 * q] = bf16_lo(v[q]);
        x[2 * q + 1] = bf16_hi(v[q]);
    }
}

template <int U>
__device__ bool rs_tile_bf16_paired(const RingParams& p, int r, int from, int k, int j, const TilePos& t,
                                    bool first, bool last, int lane, bool wait) {
    static_assert(U % 2 == 0, "two 4-element carry vectors per bf16 vector");
    const rsrc_t own = tile_view((const unsigned short*)p.src[r] + t.e0, t.len * 2);
    const rsrc_t rcv16 = tile_view((const unsigned short*)p.src[from] + t.e0, t.len * 2);
    const rsrc_t rcv32 = tile_view(p.carry + (size_t)from * p.n + t.e0, t.len * 4);
    const rsrc_t out32 = tile_view(p.carry + (size_t)r * p.n + t.e0, t.len * 4);
    const rsrc_t out16 = tile_view((unsigned short*)p.dst[r] + t.e0, t.len * 2);
    const int seen = wait ? peek_flag(p, k, from, j) : 1;
    u32x4 a[U / 2];
#pragma unroll
    for (int i = 0; i < U / 2; ++i) a[i] = ld16<POL_OWN>(own, (unsigned)(lane + i * kWave) * 16u);
    if (wait && !wait_flag(p, k, from, r, j, lane, seen)) return false;
#pragma unroll
    for (int i = 0; i < U / 2; ++i) {
        const unsigned v = (unsigned)(lane + i * kWave);                  // bf16 vector
        const unsigned c0 = (unsigned)(2 * i * kWave + lane) * 16u;      // its carry halves
        const unsigned c1 = c0 + (unsigned)kWave * 16u;
        float x[8], y[8];
        if (first) {
            bf16x8_to_f32(ld16<POL_RCV>(rcv16, v * 16u), x);
        } else {
            const u32x4 b0 = ld16<POL_RCV>(rcv32, c0), b1 = ld16<POL_RCV>(rcv32, c1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[q] = __uint_as_float(b0[q]);
                x[4 + q] = __uint_as_float(b1[q]);
            }
        }
        bf16x8_to_f32(a[i], y);
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = y[q] + x[q];
        if (last) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = pack_bf16(x[2 * q], x[2 * q + 1]);
            st16<POL_PUB>(o, out16, v * 16u);
        } else {
            u32x4 o0, o1;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                o0[q] = __float_as_uint(x[q]);
                o1[q] = __float_as_uint(x[4 + q]);
            }
            st16<POL_PUB>(o0, out32, c0);
            st16<POL_PUB>(o1, out32, c1);
        }
    }
    return true;
}

// One reduce-scatter round of tile t (position j), bf16 inputs with the fp32
// carry, from rank `from`:
//   first  : carry[r][t] = f32(src[r][t]) + f32(src[from][t])
//   middle : carry[r][t] = f32(src[r][t]) + carry[from][t]
//   last   : dst[r][t]   = bf16(f32(src[r][t]) + carry[from][t])
template <int U>
__device__ bool rs_tile_bf16_at(const RingParams& p, int r, int from, int k, int j, const TilePos& t,
                                bool first, bool last, int lane, bool wait) {
    if (carry_paired(p, t)) return rs_tile_bf16_paired<U>(p, r, from, k, j, t, first, last, lane, wait);
    const rsrc_t own = tile_view((const unsigned short*)p.src[r] + t.e0, t.len * 2);
    const rsrc_t rcv16 = tile_view((const unsigned short*)p.src[from] + t.e0, t.len * 2);
    const rsrc_t rcv32 = tile_view(p.carry + (size_t)from * p.n + t.e0, t.len * 4);
    const rsrc_t out32 = tile_view(p.carry + (size_t)r * p.n + t.e0, t.len * 4);
    const rsrc_t out16 = tile_view((unsigned short*)p.dst[r] + t.e0, t.len * 2);
    const int seen = wait ? peek_flag(p, k, from, j) : 1;
    if (p.vec_ok) {
        // lane vector v = 4 elements: 8 bytes of bf16, 16 bytes of fp32 carry
        u32x2 a[U];
#pragma unroll
        for (int i = 0; i < U; ++i) a[i] = ld8<POL_OWN>(own, (unsigned)(lane + i * kWave) * 8u);
        if (wait && !wait_flag(p, k, from, r, j, lane, seen)) return false;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const unsigned v = (unsigned)(lane + i * kWave);
            float x[4];
            if (first) {
                const u32x2 b = ld8<POL_RCV>(rcv16, v * 8u);
                x[0] = bf16_lo(b[0]); x[1] = bf16_hi(b[0]); x[2] = bf16_lo(b[1]); x[3] = bf16_hi(b[1]);
            } else {
                const u32x4 b = ld16<POL_RCV>(rcv32, v * 16u);
#pragma unroll
                for (int q = 0; q < 4; ++q) x[q] = __uint_as_float(b[q]);
            }
            x[0] = bf16_lo(a[i][0]) + x[0];
            x[1] = bf16_hi(a[i][0]) + x[1];
            x[2] = bf16_lo(a[i][1]) + x[2];
            x[3] = bf16_hi(a[i][1]) + x[3];
            if (last) {
                u32x2 o;
                o[0] = pack_bf16(x[0], x[1]);
                o[1] = pack_bf16(x[2], x[3]);
                st8<POL_PUB>(o, out16, v * 8u);
            } else {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(x[q]);
                st16<POL_PUB>(o, out32, v * 16u);
            }
        }
    } else {
        if (wait && !wait_flag(p, k, from, r, j, lane, seen)) return false;
        for (long long i = lane; i < t.len; i += kWave) {
            const unsigned o2 = (unsigned)i * 2u, o4 = (unsigned)i * 4u;
            const float recv = first ? __uint_as_float((unsigned)ld2<POL_RCV>(rcv16, o2) << 16)
                                        : __uint_as_float(ld4<POL_RCV>(rcv32, o4));
            const float x = __uint_as_float((unsigned)ld2<POL_OWN>(own, o2) << 16) + recv;
            if (last) st2<POL_PUB>((unsigned short)bf16_rne(x), out16, o2);
            else st4<POL_PUB>(__float_as_uint(x), out32, o4);
        }
    }
    return true;
}

template <int U>
__device__ __forceinline__ bool rs_tile_bf16(const RingParams& p, int r, int left, int k, int j, int lane,
                                             bool wait) {
    const TilePos t = tile_pos(p, rs_chunk(r, k, p.P), j);
    return rs_tile_bf16_at<U>(p, r, left, k, j, t, k == 0, k == p.P - 2, lane, wait);
}

// Copy one tile (len elements of ESZ bytes) from `from` to `to`; the store
// policy STORE_POL is POL_DEV when a neighbour reads the result in this launch.
template <int U, int ESZ, int LOAD_POL, int STORE_POL>
__device__ __forceinline__ void copy_tile_p(rsrc_t to, rsrc_t from, long long len, bool vec, int lane) {
    if (vec) {
        u32x4 a[U];
#pragma unroll
        for (int i = 0; i < U; ++i) a[i] = ld16<LOAD_POL>(from, (unsigned)(lane + i * kWave) * 16u);
#pragma unroll
        for (int i = 0; i < U; ++i) st16<STORE_POL>(a[i], to, (unsigned)(lane + i * kWave) * 16u);
    } else if (ESZ == 4) {
        for (long long i = lane; i < len; i += kWave)
            st4<STORE_POL>(ld4<LOAD_POL>(from, (unsigned)i * 4u), to, (unsigned)i * 4u);
    } else {
        for (long long i = lane; i < len; i += kWave)
            st2<STORE_POL>(ld2<LOAD_POL>(from, (unsigned)i * 2u), to, (unsigned)i * 2u);
    }
}
template <int U, int ESZ, int LOAD_POL>
__device__ __forceinline__ void copy_tile(rsrc_t to, rsrc_t from, long long len, bool vec,
                                          bool pub, int lane) {
    if (pub) copy_tile_p<U, ESZ, LOAD_POL, POL_PUB>(to, from, len, vec, lane);
    else copy_tile_p<U, ESZ, LOAD_POL, POL_FIN>(to, from, len, vec, lane);
}

// One all-gather round of one tile: dst[r][c] = dst[left][c].
template <int DT, int U>
__device__ bool ag_tile(const RingParams& p, int r, int left, int k, int j, int lane, bool wait) {
    constexpr int ESZ = sizeof(typename Elem<DT>::T);
    constexpr int UC = U * Elem<DT>::VPE * ESZ / 16;   // 16-byte vectors per lane per tile
    const int t = k - (p.P - 1);
    const int c = ag_chunk(r, t, p.P);
    const TilePos q = tile_pos(p, c, j);
    const long long nb = q.len * ESZ;
    // the right neighbour reads this round's result in the next round
    const bool pub = (k + 1 < p.k_end);
    const rsrc_t out = tile_view((char*)p.dst[r] + q.e0 * ESZ, nb);
    if (p.compact_src && t == 0) {
        // Place this rank's own piece (input, no wait, read by nobody else:
        // the right neighbour takes it from the input too) ...
        copy_tile<UC, ESZ, POL_OWN>(tile_view((char*)p.dst[r] + ((long long)r * p.C + q.off) * ESZ, nb),
                                     tile_view((const char*)p.src[r] + q.off * ESZ, nb),
                                     q.len, p.vec_ok, false, lane);
        // ... and take the left neighbour's piece straight from its input.
        copy_tile<UC, ESZ, POL_OWN>(out, tile_view((const char*)p.src[left] + q.off * ESZ, nb),
                                     q.len, p.vec_ok, pub, lane);
        return true;
    }
    const int seen = wait ? peek_flag(p, k, left, j) : 1;
    if (wait && !wait_flag(p, k, left, r, j, lane, seen)) return false;
    copy_tile<UC, ESZ, POL_RCV>(out, tile_view((const char*)p.dst[left] + q.e0 * ESZ, nb), q.len,
                               p.vec_ok, pub, lane);
    return true;
}

// ---------------------------------------------------------------- the kernel
__device__ __forceinline__ bool map_wave(const RingParams& p, int& r, int& w) {
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int gw = blockIdx.x * kWavesPerBlock + wid;
    const int W = p.waves_per_rank;
    if (p.map_mode == 2) {
        // Keep the whole ring chain of a tile position on one XCD: workgroups
        // are dealt to the 8 XCDs round-robin, so XCD x = blockIdx % 8 holds
        // every rank's wave for the positions w with w % 8 == x.
        const int x = blockIdx.x & 7;
        const int lw = (blockIdx.x >> 3) * kWavesPerBlock + wid;
        const int m = W >> 3;
        if (lw >= p.P * m) return false;
        r = lw % p.P;
        w = (lw / p.P) * 8 + x;
        return true;
    }
    // The P waves of one tile position are consecutive, so every prefix of
    // the dispatch order holds complete rings: progress never depends on a
    // workgroup that has not been dispatched yet.
    if (gw >= p.P * W) return false;
    r = gw % p.P;
    w = gw / p.P;
    return true;
}

template <int DT, int U>
__global__ __launch_bounds__(kBlock) void ring_step_kernel(RingParams p) {
    const WsRecord rec = ring_launch_begin(p);
    int r, w;
    if (!map_wave(p, r, w)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int left = left_of(r, p.P);
    const int rs_end = p.P - 1;
    bool checked = false;
    for (int j = w; j < p.T; j += p.waves_per_rank) {
        for (int k = p.k_begin; k < p.k_end; ++k) {
            const bool wait = (k > p.k_begin);
            bool ok;
            if (k < rs_end) {
                if constexpr (DT == DT_BF16) ok = rs_tile_bf16<U>(p, r, left, k, j, lane, wait);
                else ok = rs_tile<DT, U>(p, r, left, k, j, lane, wait);
            } else {
                if constexpr (DT == DT_F32B) ok = false;   // reduce-scatter rounds only
                else ok = ag_tile<DT, U>(p, r, left, k, j, lane, wait);
            }
            if (!ok) return;
            if (k + 1 < p.k_end) {
                if (!checked) {
                    if (!ws_ok(p.status, rec, p.ws_zero, lane)) return;
                    checked = true;
                }
                if (!(r == 0 && k + 1 == p.drop_round)) signal_flag(p, k + 1, r, j, lane);
            }
        }
    }
}

// ---------------------------------------------------------------- bidirectional reduce-scatter
// ("Pallas TPU Distributed Collectives 复习文档", section 4.)  The top half of
// every chunk (its first h elements) travels left, the bottom half right.
// Tile positions j < T_top cover the top half and are pulled from the right
// neighbour; the others cover the bottom half and are pulled from the left.
// Round k = 0 .. P-2 adds this rank's contribution to chunk (r + k + 1) mod P
// (top) or (r - k - 1) mod P (bottom); round P-1 stores the complete half of
// chunk r that arrives.  A wave waits only for the same position of round
// k-1 on the rank it pulls from, which that rank's wave of the same index
// handles earlier in its own order, so the ring groups progress exactly as
// the one-way kernel's do.
struct BidirPos {
    int from;      // the rank this tile is pulled from
    TilePos t;
};
__device__ __forceinline__ BidirPos bidir_pos(const RingParams& p, int r, int k, int j) {
    BidirPos b;
    long long lo, hi;
    int jj, c;
    if (j < p.T_top) {
        b.from = (r + 1) % p.P;
        c = (r + k + 1) % p.P;
        lo = 0;
        hi = p.h;
        jj = j;
    } else {
        b.from = (r - 1 + p.P) % p.P;
        c = ((r - k - 1) % p.P + p.P) % p.P;
        lo = p.h;
        hi = p.C;
        jj = j - p.T_top;
    }
    b.t.off = lo + (long long)jj * p.tile;
    b.t.e0 = (long long)c * p.C + b.t.off;
    b.t.len = (hi - b.t.off) < p.tile ? (hi - b.t.off) : p.tile;
    return b;
}

// Last round: the half of chunk r that rank `from` completed in round P-2
// becomes this rank's result (bf16: rounded once from the fp32 carry).
template <int DT, int U>
__device__ bool bidir_final_tile(const RingParams& p, int r, int from, int k, int j, const TilePos& t,
                                 int lane, bool wait) {
    const int seen = wait ? peek_flag(p, k, from, j) : 1;
    if (wait && !wait_flag(p, k, from, r, j, lane, seen)) return false;
    if constexpr (DT == DT_BF16) {
        const rsrc_t rcv32 = tile_view(p.carry + (size_t)from * p.n + t.e0, t.len * 4);
        const rsrc_t out16 = tile_view((unsigned short*)p.dst[r] + t.e0, t.len * 2);
        if (carry_paired(p, t)) {
#pragma unroll
            for (int i = 0; i < U / 2; ++i) {
                const unsigned c0 = (unsigned)(2 * i * kWave + lane) * 16u;
                const u32x4 b0 = ld16<POL_RCV>(rcv32, c0), b1 = ld16<POL_RCV>(rcv32, c0 + (unsigned)kWave * 16u);
                u32x4 o;
                o[0] = pack_bf16(__uint_as_float(b0[0]), __uint_as_float(b0[1]));
                o[1] = pack_bf16(__uint_as_float(b0[2]), __uint_as_float(b0[3]));
                o[2] = pack_bf16(__uint_as_float(b1[0]), __uint_as_float(b1[1]));
                o[3] = pack_bf16(__uint_as_float(b1[2]), __uint_as_float(b1[3]));
                st16<POL_FIN>(o, out16, (unsigned)(lane + i * kWave) * 16u);
            }
        } else if (p.vec_ok) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const unsigned v = (unsigned)(lane + i * kWave);
                const u32x4 b = ld16<POL_RCV>(rcv32, v * 16u);
                u32x2 o;
                o[0] = pack_bf16(__uint_as_float(b[0]), __uint_as_float(b[1]));
                o[1] = pack_bf16(__uint_as_float(b[2]), __uint_as_float(b[3]));
                st8<POL_FIN>(o, out16, v * 8u);
            }
        } else {
            for (long long i = lane; i < t.len; i += kWave)
                st2<POL_FIN>((unsigned short)bf16_rne(__uint_as_float(ld4<POL_RCV>(rcv32, (unsigned)i * 4u))),
                               out16, (unsigned)i * 2u);
        }
    } else {
        const long long nb = t.len * 4;
        copy_tile<U, 4, POL_RCV>(tile_view((char*)p.dst[r] + t.e0 * 4, nb),
                                 tile_view((const char*)p.dst[from] + t.e0 * 4, nb), t.len, p.vec_ok,
                                 false, lane);
    }
    return true;
}

template <int DT, int U>
__global__ __launch_bounds__(kBlock) void ring_bidir_kernel(RingParams p) {
    const WsRecord rec = ring_launch_begin(p);
    int r, w;
    if (!map_wave(p, r, w)) return;
    const int lane = threadIdx.x & (kWave - 1);
    if (!ws_ok(p.status, rec, p.ws_zero, lane)) return;
    for (int j = w; j < p.T; j += p.waves_per_rank) {
        for (int k = p.k_begin; k < p.k_end; ++k) {
            const bool wait = (k > p.k_begin);
            const BidirPos b = bidir_pos(p, r, k, j);
            bool ok;
            if (k < p.P - 1) {
                if constexpr (DT == DT_BF16)
                    ok = rs_tile_bf16_at<U>(p, r, b.from, k, j, b.t, k == 0, false, lane, wait);
                else
                    ok = rs_tile_at<DT, U>(p, r, b.from, k, j, b.t, k == 0, lane, wait);
            } else {
                ok = bidir_final_tile<DT, U>(p, r, b.from, k, j, b.t, lane, wait);
            }
            if (!ok) return;
            if (k + 1 < p.k_end && !(r == 0 && k + 1 == p.drop_round)) signal_flag(p, k + 1, r, j, lane);
        }
    }
}

// ---------------------------------------------------------------- circulating-input psum
// ("Pallas TPU Distributed Collectives 复习文档", section 3.)  Every rank's
// whole input travels once around the ring; each rank adds what arrives,
// x_{d-1} first and its own input last, into an accumulator that starts at
// zero.  Rank d has two receive slots.  Tile j of rank d, in one wave:
//   first send : src[d] -> slot 0 of the right neighbour; flag recv(0, right)
//   step s     : (s < P-1) flag cap(s, d): my slot (s+1) % 2 is free again
//                wait recv(s, d); load slot s % 2; add it to the accumulator
//                (s < P-1) wait cap(s, right); store the item into the right
//                neighbour's slot (s+1) % 2; flag recv(s+1, right)
//   end        : dst[d] = the accumulator
// recv(s, d) says slot s % 2 of rank d holds the item of step s; cap(s, d)
// that rank d has finished step s-1, so its slot (s+1) % 2 may be written
// (the page's capacity semaphore).  The last step's forward, which the page
// also makes, would only carry an item back to where it has been: it is left
// out.  Every flag has one reader and is cleared by it.  A wave waits on the
// rank it receives from (an earlier step) or on its right neighbour having
// started step s (which needs that neighbour's step s-1 and so on round the
// ring, ending at an earlier step of this wave), so the P waves of a tile
// position always progress.
__device__ __forceinline__ int* recv_flag(const RingParams& p, int s, int d, int j) {
    return flag_at(p, s, d, j);
}
__device__ __forceinline__ int* cap_flag(const RingParams& p, int s, int d, int j) {
    return flag_at(p, p.P + s, d, j);
}

template <int DT, int U>
__device__ bool psum_tile(const RingParams& p, int d, int j, int lane) {
    constexpr int ESZ = sizeof(typename Elem<DT>::T);
    const int P = p.P;
    const int right = (d + 1) % P;
    const long long e0 = (long long)j * p.tile;
    const long long len = (p.n - e0) < p.tile ? (p.n - e0) : p.tile;
    const long long nb = len * ESZ;
    auto slot = [&](int r, int b) {
        return tile_view((const char*)p.slots + (((size_t)r * 2 + b) * p.n + e0) * ESZ, nb);
    };
    const rsrc_t own = tile_view((const char*)p.src[d] + e0 * ESZ, nb);
    const rsrc_t out = tile_view((char*)p.dst[d] + e0 * ESZ, nb);
    const bool drop = (d == 0 && p.drop_round > 0);   // test hook (0 = off)
    auto sig = [&](int* f, int row) {
        if (!(drop && row == p.drop_round)) signal_flag(f, lane, p.check_flags, p.status, d, row, j);
    };
    auto wait = [&](int* f, int s) {
        return wait_flag(f, p.status, p.spin_limit, d, s, j, lane, peek_flag(f));
    };
    if (p.vec_ok) {
        // a lane vector is 4 elements: 16 bytes (fp32, int32) or 8 (bf16)
        float accf[U][4];
        unsigned acci[U][4];
#pragma unroll
        for (int i = 0; i < U; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                accf[i][e] = 0.0f;
                acci[i][e] = 0u;
            }
        // first send
        if constexpr (DT == DT_BF16)
            copy_tile_p<U / 2, 2, POL_OWN, POL_PUB>(slot(right, 0), own, len, true, lane);
        else
            copy_tile_p<U, 4, POL_OWN, POL_PUB>(slot(right, 0), own, len, true, lane);
        sig(recv_flag(p, 0, right, j), 0);
        for (int s = 0; s < P; ++s) {
            const bool fwd = (s < P - 1);
            if (fwd) sig(cap_flag(p, s, d, j), P + s);
            if (!wait(recv_flag(p, s, d, j), s)) return false;
            const rsrc_t in = slot(d, s & 1);
            if constexpr (DT == DT_BF16) {
                u32x2 it[U];
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    it[i] = ld8<POL_RCV>(in, (unsigned)(lane + i * kWave) * 8u);
                    accf[i][0] += bf16_lo(it[i][0]);
                    accf[i][1] += bf16_hi(it[i][0]);
                    accf[i][2] += bf16_lo(it[i][1]);
                    accf[i][3] += bf16_hi(it[i][1]);
                }
                if (fwd) {
                    if (!wait(cap_flag(p, s, right, j), s)) return false;
                    const rsrc_t o = slot(right, (s + 1) & 1);
#pragma unroll
                    for (int i = 0; i < U; ++i) st8<POL_PUB>(it[i], o, (unsigned)(lane + i * kWave) * 8u);
                    sig(recv_flag(p, s + 1, right, j), s + 1);
                }
            } else {
                u32x4 it[U];
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    it[i] = ld16<POL_RCV>(in, (unsigned)(lane + i * kWave) * 16u);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (DT == DT_F32) accf[i][e] += __uint_as_float(it[i][e]);
                        else acci[i][e] += it[i][e];
                    }
                }
                if (fwd) {
                    if (!wait(cap_flag(p, s, right, j), s)) return false;
                    const rsrc_t o = slot(right, (s + 1) & 1);
#pragma unroll
                    for (int i = 0; i < U; ++i) st16<POL_PUB>(it[i], o, (unsigned)(lane + i * kWave) * 16u);
                    sig(recv_flag(p, s + 1, right, j), s + 1);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const unsigned v = (unsigned)(lane + i * kWave);
            if constexpr (DT == DT_BF16) {
                u32x2 o;
                o[0] = pack_bf16(accf[i][0], accf[i][1]);
                o[1] = pack_bf16(accf[i][2], accf[i][3]);
                st8<POL_FIN>(o, out, v * 8u);
            } else {
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = DT == DT_F32 ? __float_as_uint(accf[i][e]) : acci[i][e];
                st16<POL_FIN>(o, out, v * 16u);
            }
        }
        return true;
    }
    // scalar path (buffers whose element count breaks 16-byte alignment):
    // one element per lane per pass; the forward re-reads the item from this
    // rank's own slot, which nobody writes before this wave flags cap(s+1, d)
    constexpr int EPL = U * 4;   // elements per lane
    unsigned acc[EPL];           // fp32 bits, or the int32 sum
#pragma unroll
    for (int i = 0; i < EPL; ++i) acc[i] = 0u;
    copy_tile_p<U, ESZ, POL_OWN, POL_PUB>(slot(right, 0), own, len, false, lane);
    sig(recv_flag(p, 0, right, j), 0);
    for (int s = 0; s < P; ++s) {
        const bool fwd = (s < P - 1);
        if (fwd) sig(cap_flag(p, s, d, j), P + s);
        if (!wait(recv_flag(p, s, d, j), s)) return false;
        const rsrc_t in = slot(d, s & 1);
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const unsigned idx = (unsigned)(lane + i * kWave);
            if constexpr (DT == DT_BF16)
                acc[i] = __float_as_uint(__uint_as_float(acc[i]) +
                                         __uint_as_float((unsigned)ld2<POL_RCV>(in, idx * 2u) << 16));
            else if constexpr (DT == DT_F32)
                acc[i] = __float_as_uint(__uint_as_float(acc[i]) + __uint_as_float(ld4<POL_RCV>(in, idx * 4u)));
            else
                acc[i] += ld4<POL_RCV>(in, idx * 4u);
        }
        if (fwd) {
            if (!wait(cap_flag(p, s, right, j), s)) return false;
            copy_tile_p<U, ESZ, POL_RCV, POL_PUB>(slot(right, (s + 1) & 1), in, len, false, lane);
            sig(recv_flag(p, s + 1, right, j), s + 1);
        }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const unsigned idx = (unsigned)(lane + i * kWave);
        if constexpr (DT == DT_BF16) st2<POL_FIN>((unsigned short)bf16_rne(__uint_as_float(acc[i])), out, idx * 2u);
        else st4<POL_FIN>(acc[i], out, idx * 4u);
    }
    return true;
}

template <int DT, int U>
__global__ __launch_bounds__(kBlock) void ring_psum_kernel(RingParams p) {
    const WsRecord rec = ring_launch_begin(p);
    int r, w;
    if (!map_wave(p, r, w)) return;
    const int lane = threadIdx.x & (kWave - 1);
    if (!ws_ok(p.status, rec, p.ws_zero, lane)) return;
    for (int j = w; j < p.T; j += p.waves_per_rank)
        if (!psum_tile<DT, U>(p, r, j, lane)) return;
}

// ---------------------------------------------------------------- copy / fill
// ---------------------------------------------------------------- low-latency rounds
// The one-way ring's rounds (same chunks, same additions in the same order)
// for calls small enough that a round's time is its latency.  The value rank
// r passes right in round k, for element o of the round's chunk, travels in
// the 8-byte word (k, r, o) of p.ll as value | 1 << 32.  The right neighbour
// polls that word until the mark is set and then clears it (it is the word's
// only reader), so a finished launch leaves every word zero.  An aligned
// 8-byte access is single-copy atomic, so a word never shows the mark with a
// stale value: LLVM's AMDGPU backend (AMDGPUUsage, the GFX942 memory model,
// which gfx950 follows) implements a monotonic atomic load or store of up to
// 64 bits as one plain load or store instruction, which is sound only
// because a naturally aligned access of that size is single-copy atomic.  With flags a round costs four trips to the device coherence
// point one after the other (the data store and its acknowledgement, the
// flag add, the poll that sees it, the data load); here two (the store, the
// poll that returns the data).  fp32 partial sums of bf16 data travel as
// fp32, bf16 values of the all-gather rounds in the low half of the value.
// The outputs go to dst as in the flag rounds: the partial sums of fp32 and
// int32 reduce-scatter rounds too, the owner's sum, every all-gather copy.
// Tile position j of a chunk covers offsets 256 j + 64 i + lane, i < 4, so
// each access instruction of a wave touches consecutive elements.  Waves
// take positions and rounds in the flag kernel's order, so the argument
// that every wave can finish is the same.
typedef unsigned long long u64;
constexpr int kLlTile = kWave * kLlVec;   // elements per tile position

// Every access goes through a buffer view of one chunk (or one round's
// words), so a lane past the chunk's end reads zeros and its stores are
// dropped by the hardware: no branch per element, and the compiler keeps
// each group of loads in flight together.
__device__ __forceinline__ rsrc_t ll_words(const RingParams& p, int k, int r) {
    return tile_view(p.ll + ((size_t)k * p.P + r) * (size_t)p.C, p.C * 8);
}
template <int DT> __device__ __forceinline__ rsrc_t ll_chunk(const void* base, long long e0, long long len) {
    constexpr int ESZ = DT == DT_BF16 ? 2 : 4;
    return tile_view((const char*)base + e0 * ESZ, len * ESZ);
}
// Element o of a view as 32 bits (bf16 zero-extended), and back.
template <int DT> __device__ __forceinline__ unsigned ll_ld(rsrc_t v, long long o) {
    if constexpr (DT == DT_BF16) return ld2<POL_PLAIN>(v, (unsigned)o * 2u);
    else return ld4<POL_PLAIN>(v, (unsigned)o * 4u);
}
template <int DT> __device__ __forceinline__ void ll_st(rsrc_t v, long long o, unsigned x) {
    if constexpr (DT == DT_BF16) st2<POL_PLAIN>((unsigned short)x, v, (unsigned)o * 2u);
    else st4<POL_PLAIN>(x, v, (unsigned)o * 4u);
}

// Rank q's input at offsets o0 + 64 i of the chunk starting at element e0,
// as the sum of its K ranges in order s = 0 .. nranges-1 (fp32).  Every
// range's loads are issued before any is added; a range past nranges is
// read through an empty view and never added (a select, not an add of
// zero, so a sum of -0 keeps its sign).
__device__ __forceinline__ void ll_ranges(const RingParams& p, int q, long long e0, long long o0,
                                          unsigned (&v)[kLlVec]) {
    float x[kLlMaxRanges][kLlVec];
#pragma unroll
    for (int s = 0; s < kLlMaxRanges; ++s) {
        const int sc = s < p.nranges ? s : 0;
        const rsrc_t in = tile_view(p.ranges + ((size_t)sc * p.P + q) * (size_t)p.n + e0,
                                    s < p.nranges ? p.C * 4 : 0);
#pragma unroll
        for (int i = 0; i < kLlVec; ++i) x[s][i] = __uint_as_float(ld4<POL_NT>(in, (unsigned)(o0 + i * kWave) * 4u));
    }
#pragma unroll
    for (int i = 0; i < kLlVec; ++i) {
        float a = x[0][i];
#pragma unroll
        for (int s = 1; s < kLlMaxRanges; ++s) a = s < p.nranges ? a + x[s][i] : a;
        v[i] = __float_as_uint(a);
    }
}

// Round k of rank r waits for the words (k - 1, from) at this lane's
// offsets o0 + 64 i (those below C: the others read as zero and count as
// ready), takes their values and clears them.  Every poll reloads all four
// words under one wait.  False if the launch is being abandoned (a timeout
// here or elsewhere).
__device__ bool ll_recv(const RingParams& p, int k, int from, long long o0, unsigned (&v)[kLlVec], int r,
                        int j, int lane) {
    const rsrc_t w = ll_words(p, k - 1, from);
    bool past[kLlVec];                     // offsets past the chunk: always ready
#pragma unroll
    for (int i = 0; i < kLlVec; ++i) past[i] = o0 + i * kWave >= p.C;
    u32x2 x[kLlVec];
    auto poll = [&] {
#pragma unroll
        for (int i = 0; i < kLlVec; ++i) x[i] = ld8<POL_DEV>(w, (unsigned)(o0 + i * kWave) * 8u);
        bool all = true;
#pragma unroll
        for (int i = 0; i < kLlVec; ++i) all = all & (past[i] | (x[i][1] != 0u));
        return all;
    };
    if (!__all(poll())) {
        const long long t0 = wall_clock64();
        unsigned spins = 0;
        for (;;) {
            __builtin_amdgcn_s_sleep(1);
            if (__all(poll())) break;
            if ((++spins & 31u) == 0) {
                if (__hip_atomic_load(&p.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
                    return false;
                if (wall_clock64() - t0 > p.spin_limit) {
                    if (lane == 0) report_timeout(p.status, r, k, j);
                    return false;
                }
            }
        }
    }
    const u32x2 zero = {0u, 0u};
#pragma unroll
    for (int i = 0; i < kLlVec; ++i) {
        v[i] = x[i][0];
        st8<POL_DEV>(zero, w, (unsigned)(o0 + i * kWave) * 8u);
    }
    return true;
}

// Pass this lane's values of round k on to the right neighbour.  With the
// check_flags debug knob every word must still be empty (each word is
// written once per launch and cleared by its one reader): a mark already
// set is recorded as RING_EPROTOCOL at (r, k + 1, j).
__device__ __forceinline__ void ll_send(const RingParams& p, int k, int r, long long o0,
                                        const unsigned (&v)[kLlVec], int j, int lane) {
    const rsrc_t w = ll_words(p, k, r);
    if (p.check_flags) {
        bool busy = false;
#pragma unroll
        for (int i = 0; i < kLlVec; ++i) busy |= ld8<POL_DEV>(w, (unsigned)(o0 + i * kWave) * 8u)[1] != 0u;
        if (__any(busy) && lane == 0) report_error(p.status, RING_EPROTOCOL, r, k + 1, j);
    }
#pragma unroll
    for (int i = 0; i < kLlVec; ++i) {
        const u32x2 x = {v[i], 1u};
        st8<POL_DEV>(x, w, (unsigned)(o0 + i * kWave) * 8u);
    }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void ring_ll_kernel(RingParams p) {
    const WsRecord rec = ring_launch_begin(p);
    int r, w;
    if (!map_wave(p, r, w)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int P = p.P;
    const int left = left_of(r, P);
    const long long C = p.C;
    bool checked = false;
    for (int j = w; j < p.T; j += p.waves_per_rank) {
        const long long o0 = (long long)j * kLlTile + lane;
        for (int k = p.k_begin; k < p.k_end; ++k) {
            const bool send = k + 1 < p.k_end && !(r == 0 && k + 1 == p.drop_round);
            unsigned v[kLlVec];
            if (k < P - 1) {
                // reduce-scatter round s = k: chunk (r - k - 2) mod P
                const long long e0 = (long long)rs_chunk(r, k, P) * C;
                const bool summed = DT == DT_F32B && p.nranges > 0;   // inputs as sums of K ranges
                unsigned a[kLlVec];
                if (summed) {
                    ll_ranges(p, r, e0, o0, a);
                } else {
                    const rsrc_t own = ll_chunk<DT>(p.src[r], e0, C);
#pragma unroll
                    for (int i = 0; i < kLlVec; ++i) a[i] = ll_ld<DT>(own, o0 + i * kWave);
                }
                if (k == p.k_begin) {   // the left neighbour's input: complete before the launch
                    if (summed) {
                        ll_ranges(p, left, e0, o0, v);
                    } else {
                        const rsrc_t in = ll_chunk<DT>(p.src[left], e0, C);
#pragma unroll
                        for (int i = 0; i < kLlVec; ++i) {
                            const unsigned x = ll_ld<DT>(in, o0 + i * kWave);
                            v[i] = DT == DT_BF16 ? x << 16 : x;
                        }
                    }
                } else if (!ll_recv(p, k, left, o0, v, r, j, lane)) {
                    return;
                }
#pragma unroll
                for (int i = 0; i < kLlVec; ++i) {
                    if constexpr (DT == DT_I32) v[i] = v[i] + a[i];
                    else if constexpr (DT == DT_BF16)
                        v[i] = __float_as_uint(__uint_as_float(v[i]) + __uint_as_float(a[i] << 16));
                    else v[i] = __float_as_uint(__uint_as_float(v[i]) + __uint_as_float(a[i]));
                }
                const bool last = k == P - 2;   // this rank owns the chunk
                const rsrc_t out = ll_chunk<DT>(p.dst[r], e0, C);
                if constexpr (DT == DT_BF16) {
                    if (last) {
#pragma unroll
                        for (int i = 0; i < kLlVec; ++i) {
                            v[i] = bf16_rne(__uint_as_float(v[i]));   // the all-gather passes bf16 on
                            ll_st<DT>(out, o0 + i * kWave, v[i]);
                        }
                    }
                } else if constexpr (DT == DT_F32B) {
                    if (last) {
                        const rsrc_t o16 = tile_view(p.out16[r], C * 2);
#pragma unroll
                        for (int i = 0; i < kLlVec; ++i)
                            st2<POL_PLAIN>((unsigned short)bf16_rne(__uint_as_float(v[i])), o16,
                                           (unsigned)(o0 + i * kWave) * 2u);
                    } else if (!summed) {   // partial sums (unspecified outputs; none with ranges)
#pragma unroll
                        for (int i = 0; i < kLlVec; ++i) ll_st<DT>(out, o0 + i * kWave, v[i]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < kLlVec; ++i) ll_st<DT>(out, o0 + i * kWave, v[i]);
                }
            } else {
                // all-gather round t = k - (P - 1): chunk (r - t - 1) mod P
                const int t = k - (P - 1);
                const long long e0 = (long long)ag_chunk(r, t, P) * C;
                if (k == p.k_begin) {   // inputs, complete before the launch
                    if (p.compact_src) {   // place this rank's own piece, take the left one's
                        const rsrc_t mine = ll_chunk<DT>(p.src[r], 0, C);
                        const rsrc_t place = ll_chunk<DT>(p.dst[r], (long long)r * C, C);
                        const rsrc_t in = ll_chunk<DT>(p.src[left], 0, C);
#pragma unroll
                        for (int i = 0; i < kLlVec; ++i) {
                            ll_st<DT>(place, o0 + i * kWave, ll_ld<DT>(mine, o0 + i * kWave));
                            v[i] = ll_ld<DT>(in, o0 + i * kWave);
                        }
                    } else {
                        const rsrc_t in = ll_chunk<DT>(p.dst[left], e0, C);
#pragma unroll
                        for (int i = 0; i < kLlVec; ++i) v[i] = ll_ld<DT>(in, o0 + i * kWave);
                    }
                } else if (!ll_recv(p, k, left, o0, v, r, j, lane)) {
                    return;
                }
                const rsrc_t out = ll_chunk<DT>(p.dst[r], e0, C);
#pragma unroll
                for (int i = 0; i < kLlVec; ++i) ll_st<DT>(out, o0 + i * kWave, v[i]);
            }
            if (k + 1 < p.k_end && !checked) {
                if (!ws_ok(p.status, rec, p.ws_zero, lane)) return;
                checked = true;
            }
            if (send) ll_send(p, k, r, o0, v, j, lane);
        }
    }
}

__global__ __launch_bounds__(kBlock) void fill_zero_kernel(unsigned* p, long long words, long long tail_bytes) {
    const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long nth = (long long)gridDim.x * blockDim.x;
    for (long long i = tid; i < words; i += nth) p[i] = 0u;
    if (tid < tail_bytes) ((unsigned char*)(p + words))[tid] = 0;
}

// ---------------------------------------------------------------- launchers
struct PtrTables {
    const void* src[RING_MAX_RANKS];
    void* dst[RING_MAX_RANKS];
};

// dst[r] = src[(r - shift) mod P], `bytes` per rank; blockIdx.y = rank.  The
// pointer tables travel by value in the kernel-argument segment.
__global__ __launch_bounds__(kBlock) void copy_kernel_tab(PtrTables t, int P, long long bytes,
                                                          int shift, int vec) {
    const int r = blockIdx.y;
    const int from = ((r - shift) % P + P) % P;
    const char* s = (const char*)t.src[from];
    char* d = (char*)t.dst[r];
    const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long nth = (long long)gridDim.x * blockDim.x;
    if (vec) {
        // every byte is read and written once: both stream past the caches
        const long long nv = bytes / 16;
        const u32x4* sv = (const u32x4*)s;
        u32x4* dv = (u32x4*)d;
        long long i = tid;
        for (; i + 3 * nth < nv; i += 4 * nth) {
            u32x4 a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = __builtin_nontemporal_load(&sv[i + u * nth]);
#pragma unroll
            for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(a[u], &dv[i + u * nth]);
        }
        for (; i < nv; i += nth) __builtin_nontemporal_store(__builtin_nontemporal_load(&sv[i]), &dv[i]);
        for (long long b = nv * 16 + tid; b < bytes; b += nth) d[b] = s[b];
    } else {
        for (long long b = tid; b < bytes; b += nth) d[b] = s[b];
    }
}

hipError_t launch_copy(const void* const* src, void* const* dst, int P, size_t bytes, int shift,
                       hipStream_t s) {
    PtrTables t;
    int vec = 1;
    for (int r = 0; r < P; ++r) {
        t.src[r] = src[r];
        t.dst[r] = dst[r];
        if (((uintptr_t)src[r] | (uintptr_t)dst[r]) & 15) vec = 0;
    }
    const DevInfo di = dev_info();
    // one block per CU spread over the ranks, 4 x 16 bytes in flight per
    // lane: more in flight made the copy slower (4.6 against 6.2 TB/s at four
    // blocks per CU), the memory system serving fewer streams better
    long long per_rank = ((long long)di.cus + P - 1) / P;
    const long long need = (long long)((bytes + 16 * kBlock * 4 - 1) / (16 * kBlock * 4));
    if (per_rank > need) per_rank = need;
    if (per_rank < 1) per_rank = 1;
    hipLaunchKernelGGL(copy_kernel_tab, dim3((unsigned)per_rank, (unsigned)P), dim3(kBlock), 0, s,
                       t, P, (long long)bytes, shift, vec);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    const long long words = (long long)(bytes / 4);
    const long long tail = (long long)(bytes % 4);
    long long blocks = (words + kBlock - 1) / kBlock;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(kBlock), 0, s,
                       (unsigned*)p, words, tail);
    return hipGetLastError();
}

template <int DT, int U>
static hipError_t launch_ring_t(RingParams& prm, int grid, hipStream_t s) {
    if constexpr (DT == DT_F32B) {   // the one-way reduce-scatter only
        hipLaunchKernelGGL((ring_step_kernel<DT, U>), dim3(grid), dim3(kBlock), 0, s, prm);
    } else {
        if (prm.psum)
            hipLaunchKernelGGL((ring_psum_kernel<DT, U>), dim3(grid), dim3(kBlock), 0, s, prm);
        else if (prm.bidir)
            hipLaunchKernelGGL((ring_bidir_kernel<DT, U>), dim3(grid), dim3(kBlock), 0, s, prm);
        else
            hipLaunchKernelGGL((ring_step_kernel<DT, U>), dim3(grid), dim3(kBlock), 0, s, prm);
    }
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_ring_dt(RingParams& prm, int tile_vecs, int grid, hipStream_t s) {
    switch (tile_vecs) {
        case 4: return launch_ring_t<DT, 4>(prm, grid, s);
        case 8: return launch_ring_t<DT, 8>(prm, grid, s);
        case 16: return launch_ring_t<DT, 16>(prm, grid, s);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, int U>
static int blocks_per_cu_t(int kind) {
    int nb = 0;
    if constexpr (DT == DT_F32B) {   // the one-way reduce-scatter only
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ring_step_kernel<DT, U>, kBlock, 0);
        return e == hipSuccess ? nb : 0;
    } else {
        const hipError_t e =
            kind == 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ring_psum_kernel<DT, U>, kBlock, 0)
            : kind == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ring_bidir_kernel<DT, U>, kBlock, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ring_step_kernel<DT, U>, kBlock, 0);
        return e == hipSuccess ? nb : 0;
    }
}

template <int DT>
static int blocks_per_cu_dt(int tile_vecs, int kind) {
    switch (tile_vecs) {
        case 4: return blocks_per_cu_t<DT, 4>(kind);
        case 8: return blocks_per_cu_t<DT, 8>(kind);
        case 16: return blocks_per_cu_t<DT, 16>(kind);
        default: return 0;
    }
}

template <int DT>
static int blocks_per_cu_ll() {
    int nb = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ring_ll_kernel<DT>, kBlock, 0) == hipSuccess ? nb : 0;
}

int ring_blocks_per_cu(int dtype, int tile_vecs, int kind) {
    if (kind == 3) {
        switch (dtype) {
            case RING_F32: return blocks_per_cu_ll<DT_F32>();
            case kDtF32Bf16Out: return blocks_per_cu_ll<DT_F32B>();
            case RING_I32: return blocks_per_cu_ll<DT_I32>();
            case RING_BF16: return blocks_per_cu_ll<DT_BF16>();
            default: return 0;
        }
    }
    switch (dtype) {
        case RING_F32: return blocks_per_cu_dt<DT_F32>(tile_vecs, kind);
        case kDtF32Bf16Out: return blocks_per_cu_dt<DT_F32B>(tile_vecs, kind);
        case RING_I32: return blocks_per_cu_dt<DT_I32>(tile_vecs, kind);
        case RING_BF16: return blocks_per_cu_dt<DT_BF16>(tile_vecs, kind);
        default: return 0;
    }
}

template <int DT>
static hipError_t launch_ll(RingParams& prm, int grid, hipStream_t s) {
    hipLaunchKernelGGL((ring_ll_kernel<DT>), dim3(grid), dim3(kBlock), 0, s, prm);
    return hipGetLastError();
}

hipError_t launch_ring(RingParams& prm, int dtype, int tile_vecs, int grid, hipStream_t s) {
    if (prm.ll) {
        switch (dtype) {
            case RING_F32: return launch_ll<DT_F32>(prm, grid, s);
            case kDtF32Bf16Out: return launch_ll<DT_F32B>(prm, grid, s);
            case RING_I32: return launch_ll<DT_I32>(prm, grid, s);
            case RING_BF16: return launch_ll<DT_BF16>(prm, grid, s);
            default: return hipErrorInvalidValue;
        }
    }
    switch (dtype) {
        case RING_F32: return launch_ring_dt<DT_F32>(prm, tile_vecs, grid, s);
        case kDtF32Bf16Out: return launch_ring_dt<DT_F32B>(prm, tile_vecs, grid, s);
        case RING_I32: return launch_ring_dt<DT_I32>(prm, tile_vecs, grid, s);
        case RING_BF16: return launch_ring_dt<DT_BF16>(prm, tile_vecs, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ringc

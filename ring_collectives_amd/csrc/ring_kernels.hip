// ring_kernels.hip -- gfx950 kernels of the ring collectives.
//
//   * copy_kernel_tab   : ppermute (dst[r] = src[(r - shift) mod P]), and the
//                         plain copies of the P = 1 cases.
//   * ring_step_kernel  : the persistent chunk-step kernel that runs the ring
//                         reduce-scatter and all-gather rounds for every
//                         virtual rank at once.
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
// round k-1".  The producer wave makes its stores visible at agent scope
// (release fence: L2 write-back so other XCDs see them) and adds 1 to the flag;
// the consumer wave polls the flag until it is >= 1, then takes an
// agent-scope acquire fence (L2/L1 invalidate) before it loads its
// neighbour's data.  Each flag is set by one wave and read by one wave per
// launch, so the reader clears it after use and a finished launch leaves the
// table zeroed for the next one.
//
// Work assignment.  Each rank gets `waves_per_rank` waves; wave w of rank r
// takes tile positions j = w, w + W, w + 2W, ... and for each position runs
// every round k in order.  A wave only ever waits for (k-1, left, j), which
// belongs to the left rank's wave with the same w and an earlier place in
// that wave's own order (same j, smaller k), so as long as all waves are
// resident at once the dependencies always drain: the host sizes the grid
// from the occupancy query so that they are.  A watchdog bounds every wait.
#include "ring_internal.h"

#include <hip/hip_runtime.h>

namespace ringc {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F32 = RING_F32, DT_BF16 = RING_BF16, DT_I32 = RING_I32 };

__device__ __forceinline__ int left_of(int r, int P) { return (r - 1 + P) % P; }
__device__ __forceinline__ int rs_chunk(int r, int s, int P) { return (r - s - 2 + 2 * P) % P; }
__device__ __forceinline__ int ag_chunk(int r, int t, int P) { return (r - t - 1 + P) % P; }

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

__device__ void report_timeout(const RingParams& p, int r, int k, int j) {
    int expected = 0;
    if (__hip_atomic_compare_exchange_strong(&p.status->code, &expected, (int)RING_ETIMEOUT,
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)) {
        int info = (r & 0xFF) | ((k & 0xFF) << 8) | ((j < 32767 ? j : 32767) << 16);
        __hip_atomic_store(&p.status->info, info, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Wait until flag (k, left, j) is set, then acquire.  Returns false if the
// launch is being abandoned (this wave timed out, or another one did).
__device__ bool wait_flag(const RingParams& p, int k, int left, int r, int j, int lane) {
    int* f = flag_at(p, k, left, j);
    if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < 1) {
        const long long t0 = wall_clock64();
        unsigned spins = 0;
        while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < 1) {
            __builtin_amdgcn_s_sleep(2);
            if ((++spins & 31u) == 0) {
                if (__hip_atomic_load(&p.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
                    return false;
                if (wall_clock64() - t0 > p.spin_limit) {
                    if (lane == 0) report_timeout(p, r, k, j);
                    return false;
                }
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // This wave is the flag's only reader in this launch: clear it for the next.
    if (lane == 0) __hip_atomic_store(f, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Publish this wave's stores of round k-1 and set flag (k, r, j).
__device__ __forceinline__ void signal_flag(const RingParams& p, int k, int r, int j, int lane) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    if (lane == 0)
        __hip_atomic_fetch_add(flag_at(p, k, r, j), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- tile bodies
// Element types.
template <int DT> struct Elem;
template <> struct Elem<DT_F32> { typedef float T; static constexpr int VPE = 4; };
template <> struct Elem<DT_I32> { typedef int T; static constexpr int VPE = 4; };
template <> struct Elem<DT_BF16> { typedef unsigned short T; static constexpr int VPE = 8; };

template <int DT> __device__ __forceinline__ u32x4 add_vec(u32x4 a, u32x4 b);
template <> __device__ __forceinline__ u32x4 add_vec<DT_F32>(u32x4 a, u32x4 b) {
    f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
    return __builtin_bit_cast(u32x4, x + y);
}
template <> __device__ __forceinline__ u32x4 add_vec<DT_I32>(u32x4 a, u32x4 b) {
    return a + b;  // wraps modulo 2^32
}

template <int DT> __device__ __forceinline__ void add_scalar(const void* own, const void* rcv,
                                                              void* out, long long i);
template <> __device__ __forceinline__ void add_scalar<DT_F32>(const void* own, const void* rcv,
                                                                void* out, long long i) {
    ((float*)out)[i] = ((const float*)own)[i] + ((const float*)rcv)[i];
}
template <> __device__ __forceinline__ void add_scalar<DT_I32>(const void* own, const void* rcv,
                                                                void* out, long long i) {
    ((unsigned*)out)[i] = ((const unsigned*)own)[i] + ((const unsigned*)rcv)[i];
}

// One reduce-scatter round of one tile, fp32 / int32.
template <int DT, int U>
__device__ bool rs_tile(const RingParams& p, int r, int left, int k, int j, int lane, bool wait) {
    typedef typename Elem<DT>::T T;
    const int s = k;
    const int c = rs_chunk(r, s, p.P);
    const long long off = (long long)j * p.tile;
    const long long e0 = (long long)c * p.C + off;
    const long long len = (p.C - off) < p.tile ? (p.C - off) : p.tile;
    const T* own = (const T*)p.src[r] + e0;
    const T* rcv = (s == 0 ? (const T*)p.src[left] : (const T*)p.dst[left]) + e0;
    T* out = (T*)p.dst[r] + e0;
    if (p.vec_ok && len == p.tile) {
        u32x4 a[U], b[U];
        const u32x4* ov = (const u32x4*)own;
#pragma unroll
        for (int i = 0; i < U; ++i) a[i] = ov[lane + i * kWave];
        if (wait && !wait_flag(p, k, left, r, j, lane)) return false;
        const u32x4* rv = (const u32x4*)rcv;
#pragma unroll
        for (int i = 0; i < U; ++i) b[i] = rv[lane + i * kWave];
        u32x4* dv = (u32x4*)out;
#pragma unroll
        for (int i = 0; i < U; ++i) dv[lane + i * kWave] = add_vec<DT>(a[i], b[i]);
    } else {
        if (wait && !wait_flag(p, k, left, r, j, lane)) return false;
        for (long long i = lane; i < len; i += kWave) add_scalar<DT>(own, rcv, out, i);
    }
    return true;
}

// One reduce-scatter round of one tile, bf16 inputs with the fp32 carry.
template <int U>
__device__ bool rs_tile_bf16(const RingParams& p, int r, int left, int k, int j, int lane, bool wait) {
    const int s = k;
    const int c = rs_chunk(r, s, p.P);
    const bool last = (s == p.P - 2);
    const long long off = (long long)j * p.tile;
    const long long e0 = (long long)c * p.C + off;
    const long long len = (p.C - off) < p.tile ? (p.C - off) : p.tile;
    const unsigned short* own = (const unsigned short*)p.src[r] + e0;
    const unsigned short* rcv16 = (const unsigned short*)p.src[left] + e0;   // round 0
    const float* rcv32 = p.carry + (size_t)left * p.n + e0;                  // rounds >= 1
    float* out32 = p.carry + (size_t)r * p.n + e0;
    unsigned short* out16 = (unsigned short*)p.dst[r] + e0;
    if (p.vec_ok && len == p.tile) {
        u32x4 a[U];
#pragma unroll
        for (int i = 0; i < U; ++i) a[i] = ((const u32x4*)own)[lane + i * kWave];
        if (wait && !wait_flag(p, k, left, r, j, lane)) return false;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const long long v = lane + i * kWave;   // vector of 8 elements
            float x[8];
            if (s == 0) {
                const u32x4 b = ((const u32x4*)rcv16)[v];
#pragma unroll
                for (int q = 0; q < 4; ++q) { x[2 * q] = bf16_lo(b[q]); x[2 * q + 1] = bf16_hi(b[q]); }
            } else {
                const f32x4 b0 = ((const f32x4*)rcv32)[2 * v];
                const f32x4 b1 = ((const f32x4*)rcv32)[2 * v + 1];
#pragma unroll
                for (int q = 0; q < 4; ++q) { x[q] = b0[q]; x[4 + q] = b1[q]; }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                x[2 * q] = bf16_lo(a[i][q]) + x[2 * q];
                x[2 * q + 1] = bf16_hi(a[i][q]) + x[2 * q + 1];
            }
            if (last) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = pack_bf16(x[2 * q], x[2 * q + 1]);
                ((u32x4*)out16)[v] = o;
            } else {
                ((f32x4*)out32)[2 * v] = f32x4{x[0], x[1], x[2], x[3]};
                ((f32x4*)out32)[2 * v + 1] = f32x4{x[4], x[5], x[6], x[7]};
            }
        }
    } else {
        if (wait && !wait_flag(p, k, left, r, j, lane)) return false;
        for (long long i = lane; i < len; i += kWave) {
            const float recv = (s == 0) ? __uint_as_float((unsigned)rcv16[i] << 16) : rcv32[i];
            const float x = __uint_as_float((unsigned)own[i] << 16) + recv;
            if (last) out16[i] = (unsigned short)bf16_rne(x);
            else out32[i] = x;
        }
    }
    return true;
}

// Copy `len` elements of `esz` bytes; vector path when aligned and full.
template <int U>
__device__ __forceinline__ void copy_elems(void* dst, const void* src, long long len, int esz,
                                           bool full_vec, int lane) {
    if (full_vec) {
        u32x4 a[U];
#pragma unroll
        for (int i = 0; i < U; ++i) a[i] = ((const u32x4*)src)[lane + i * kWave];
#pragma unroll
        for (int i = 0; i < U; ++i) ((u32x4*)dst)[lane + i * kWave] = a[i];
    } else if (esz == 4) {
        for (long long i = lane; i < len; i += kWave) ((unsigned*)dst)[i] = ((const unsigned*)src)[i];
    } else {
        for (long long i = lane; i < len; i += kWave)
            ((unsigned short*)dst)[i] = ((const unsigned short*)src)[i];
    }
}

// One all-gather round of one tile (a copy from the left neighbour).
template <int DT, int U>
__device__ bool ag_tile(const RingParams& p, int r, int left, int k, int j, int lane, bool wait) {
    constexpr int ESZ = sizeof(typename Elem<DT>::T);
    const int t = k - (p.P - 1);
    const int c = ag_chunk(r, t, p.P);
    const long long off = (long long)j * p.tile;
    const long long len = (p.C - off) < p.tile ? (p.C - off) : p.tile;
    const bool full_vec = p.vec_ok && len == p.tile;
    char* out = (char*)p.dst[r] + ((long long)c * p.C + off) * ESZ;
    if (p.compact_src && t == 0) {
        // Place this rank's own piece (input, no wait needed) ...
        copy_elems<U>((char*)p.dst[r] + ((long long)r * p.C + off) * ESZ,
                      (const char*)p.src[r] + off * ESZ, len, ESZ, full_vec, lane);
        // ... and take the left neighbour's piece straight from its input.
        copy_elems<U>(out, (const char*)p.src[left] + off * ESZ, len, ESZ, full_vec, lane);
        return true;
    }
    if (wait && !wait_flag(p, k, left, r, j, lane)) return false;
    copy_elems<U>(out, (const char*)p.dst[left] + ((long long)c * p.C + off) * ESZ, len, ESZ,
                  full_vec, lane);
    return true;
}

// ---------------------------------------------------------------- the kernel
__device__ __forceinline__ bool map_wave(const RingParams& p, int& r, int& w) {
    const int wid = threadIdx.x / kWave;
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
    if (gw >= p.P * W) return false;
    if (p.map_mode == 1) { r = gw / W; w = gw % W; }
    else { r = gw % p.P; w = gw / p.P; }
    return true;
}

template <int DT, int U>
__global__ __launch_bounds__(kBlock) void ring_step_kernel(RingParams p) {
    int r, w;
    if (!map_wave(p, r, w)) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int left = left_of(r, p.P);
    const int rs_end = p.P - 1;
    for (int j = w; j < p.T; j += p.waves_per_rank) {
        for (int k = p.k_begin; k < p.k_end; ++k) {
            const bool wait = (k > p.k_begin);
            bool ok;
            if (k < rs_end) {
                if constexpr (DT == DT_BF16) ok = rs_tile_bf16<U>(p, r, left, k, j, lane, wait);
                else ok = rs_tile<DT, U>(p, r, left, k, j, lane, wait);
            } else {
                ok = ag_tile<DT, U>(p, r, left, k, j, lane, wait);
            }
            if (!ok) return;
            if (k + 1 < p.k_end && !(r == 0 && k + 1 == p.drop_round))
                signal_flag(p, k + 1, r, j, lane);
        }
    }
}

// ---------------------------------------------------------------- copy / fill
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
        const long long nv = bytes / 16;
        const u32x4* sv = (const u32x4*)s;
        u32x4* dv = (u32x4*)d;
        long long i = tid;
        for (; i + 3 * nth < nv; i += 4 * nth) {
            u32x4 a0 = sv[i], a1 = sv[i + nth], a2 = sv[i + 2 * nth], a3 = sv[i + 3 * nth];
            dv[i] = a0; dv[i + nth] = a1; dv[i + 2 * nth] = a2; dv[i + 3 * nth] = a3;
        }
        for (; i < nv; i += nth) dv[i] = sv[i];
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
    // about 4 resident blocks per CU spread over the ranks
    long long per_rank = (4LL * di.cus + P - 1) / P;
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
    hipLaunchKernelGGL((ring_step_kernel<DT, U>), dim3(grid), dim3(kBlock), 0, s, prm);
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

template <int DT>
static int blocks_per_cu_dt(int tile_vecs) {
    int nb = 0;
    hipError_t e = hipErrorInvalidValue;
    switch (tile_vecs) {
        case 4: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ring_step_kernel<DT, 4>, kBlock, 0); break;
        case 8: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ring_step_kernel<DT, 8>, kBlock, 0); break;
        case 16: e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, ring_step_kernel<DT, 16>, kBlock, 0); break;
    }
    return e == hipSuccess ? nb : 0;
}

int ring_blocks_per_cu(int dtype, int tile_vecs) {
    switch (dtype) {
        case RING_F32: return blocks_per_cu_dt<DT_F32>(tile_vecs);
        case RING_I32: return blocks_per_cu_dt<DT_I32>(tile_vecs);
        case RING_BF16: return blocks_per_cu_dt<DT_BF16>(tile_vecs);
        default: return 0;
    }
}

hipError_t launch_ring(RingParams& prm, int dtype, int tile_vecs, int grid, hipStream_t s) {
    switch (dtype) {
        case RING_F32: return launch_ring_dt<DT_F32>(prm, tile_vecs, grid, s);
        case RING_I32: return launch_ring_dt<DT_I32>(prm, tile_vecs, grid, s);
        case RING_BF16: return launch_ring_dt<DT_BF16>(prm, tile_vecs, grid, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace ringc

// ag_gemm.hip -- all-gather + GEMM with tile-level overlap.
//
// Rank q holds row block q of A (A_shard[q], M/P x K bf16) and its own B_q
// (K x N bf16).  The ranks all-gather the row blocks around the ring into
// A_full[q] (M x K; chunk c = rows [c M/P, (c+1) M/P)) and every rank computes
// C_q = A_full @ B_q in fp32.  That is the all-gather-matmul of "TPU 与分布式
// 通信原语" (collective matmul: gather the blocks of x, multiply by the local
// weight), overlapped as the "AllGather + GEMM 重叠" pattern of
// "Triton-distributed 语义": the GEMM tiles of a block start as soon as the
// block has arrived, and every rank starts on its local block (the
// threadblock swizzle of the same page, "线程块交织").
//
// Schedule.  Phase f = 0 .. P-1 handles chunk c = (q - f) mod P, the order in
// which the ring delivers the blocks (round t of the ring all-gather brings
// chunk (q - t - 1) mod P from the left neighbour), local block first.  The
// tiles of chunk c read its rows from where they already are: phase 0 from
// A_shard[q], phase 1 from A_shard[left] (the left rank's own block), phase
// f >= 2 from A_full[left], which the left rank's phase f - 1 tiles wrote.
// Forwarding rides on those reads: the tile at column position tc of a
// 256-row panel copies the K range [tc K / tn, (tc + 1) K / tn) of the
// panel's rows (tn column tiles) from the LDS stages its K loop brings in
// anyway into A_full[q], and flags that when its K loop is done, so the tn
// tiles of a panel forward the whole panel once, with no loads of their own.
// A tile of phase f >= 2 starts once the left rank's tn phase f - 1 tiles of
// its panel have flagged.
//
// Progress.  A phase-f tile waits only for phase f - 1 tiles of the left
// rank, and every workgroup finishes its tiles of phase f - 1 before it
// starts phase f; so by induction on f every tile finishes, provided every
// workgroup gets to run (the grid is sized for the CUs; beside another
// kernel the rest start as its workgroups finish).  A flag has the tn tiles
// of the right rank's panel for readers, so readers leave it set and the last
// workgroup to finish clears the table for the next call.
#include "gemm_core.h"

#include <hip/hip_runtime.h>
#include <string.h>

namespace ringc {

struct AgGemmParams {
    const unsigned short* As[RING_MAX_RANKS];   // rank q's block of A, (M / P) x K
    const unsigned short* B[RING_MAX_RANKS];    // K x N
    unsigned short* Af[RING_MAX_RANKS];         // gathered A, M x K
    void* C[RING_MAX_RANKS];                    // M x N: fp32, or bf16 (the MLP's activation)
    int* flags;                                 // [P phases][P ranks][tpc], kFlagStride apart
    int* done;                                  // workgroups finished (clears the flags)
    Status* status;
    long long spin_limit;
    int P, M, N, K;
    int tm_chunk;                               // 256-row panels per chunk
    int tn;                                     // column tiles (N / BN)
    int tpc;                                    // tiles per chunk
    int groups;                                 // workgroups per rank
    int nflags;                                 // flags in the table
    int drop_round;                             // test hook: rank 0 never flags this phase (0 = off)
    int gelu_bf16;                              // C is bf16(gelu(bf16(product))), else fp32
    WsSpan ws_zero, ws_data;                    // flags that must start zero; data left behind
    int check_flags;                            // debug: each flag must be 0 when it is set
};

__device__ __forceinline__ int* ag_flag(const AgGemmParams& p, int f, int q, int pos) {
    return p.flags + (((size_t)f * p.P + q) * p.tpc + pos) * kFlagStride;
}

// K range [k0, k1) of the panel that column tile tc forwards (multiples of
// 8 elements, so whole 16-byte pieces; the tn ranges tile [0, K)).
__device__ __forceinline__ void forward_range(const AgGemmParams& p, int tc, int& k0, int& k1) {
    const int k8 = p.K / 8;
    k0 = (int)(((long long)tc * k8) / p.tn) * 8;
    k1 = (int)(((long long)(tc + 1) * k8) / p.tn) * 8;
}

// The K-loop hook that forwards: at the first step of each A stage that
// overlaps [k0, k1), the wave copies its kRows rows of the stage (64 columns,
// 128 bytes a row, read back from the swizzled LDS buffer) into the panel's
// rows of A_full[q], 8 rows per 16-byte-per-lane store; columns outside the
// range get an offset past the end of the view, which drops them.
template <class G>
struct ForwardHook {
    static constexpr bool kActive = true;
    static constexpr int kRows = kBM / G::NW;     // rows of a stage this wave copies
    static constexpr int kStores = kRows / 8;     // 16-byte stores per lane and stage
    const unsigned short* lds;
    rsrc_t dv;            // the panel's rows of A_full[q], all K columns
    unsigned dst_lane;    // byte offset of the lane's piece, row 0 of its rows, column 0
    unsigned row8;        // bytes of 8 rows
    unsigned lds_row;     // LDS byte offset of the lane's row within an A buffer
    int chunk;            // the lane's 16-byte piece of a row (columns 8 chunk ..)
    int swz0;             // (row >> 1) & 7 of the lane's first row
    int k0, k1;
    __device__ __forceinline__ void begin() {}
    __device__ __forceinline__ void end(int) {}
    __device__ __forceinline__ int ops(int t) const {
        if (t % G::R) return 0;
        const int kb = (t / G::R) * G::BKA;
        return kb < k1 && kb + G::BKA > k0 ? kStores : 0;
    }
    __device__ __forceinline__ void issue(int t) {
        const int st = t / G::R;
        const int kb = st * G::BKA;
        const int k = kb + 8 * chunk;
        const bool in = k >= k0 && k < k1;
        const unsigned abuf = (unsigned)((st & 1) * G::kStageA);
#pragma unroll
        for (int i = 0; i < kStores; ++i) {
            // row kRows wave + 8 i + lane / 8: its swizzle is swz0 + 4 i (mod 8)
            const int sw = (swz0 + 4 * i) & 7;
            const u32x4 v = *(const u32x4*)((const char*)lds + abuf + lds_row + (unsigned)(i * 8 * G::kARowBytes) +
                                            (unsigned)((chunk ^ sw) * 16));
            const unsigned off = in ? dst_lane + (unsigned)i * row8 + (unsigned)(kb * 2) : 0x80000000u;
            st16<POL_DEV>(v, dv, off);
        }
    }
    __device__ __forceinline__ void init(const unsigned short* l, int lane, int wave) {
        lds = l;
        const int row = kRows * wave + lane / 8;
        lds_row = (unsigned)(row * G::kARowBytes);
        chunk = lane & 7;
        swz0 = (row >> 1) & 7;
    }
    // the panel: rows (element (0, 0) at `panel`, row stride K) and this
    // tile's range
    __device__ __forceinline__ void at(unsigned short* panel, int K, int lane, int wave, int a, int b) {
        dv = tile_view(panel, (long long)kBM * K * 2);
        dst_lane = (unsigned)(((kRows * wave + lane / 8) * K + 8 * (lane & 7)) * 2);
        row8 = (unsigned)(8 * K * 2);
        k0 = a;
        k1 = b;
    }
};

// Wave 0 waits until flags f0, f0 + kFlagStride, ... (n of them) are all set,
// one lane per flag, 64 at a time, so a panel's flags cost one round trip
// to the coherence point rather than one each; the workgroup follows it
// through an LDS-only barrier, which leaves this wave's earlier output stores
// in flight (nothing in the launch reads them).  The other waves' loads of
// the flagged rows are device-scope and issued after the barrier.  Returns
// false (for every wave) if the launch is being abandoned: a wave that gives
// up has recorded the timeout in the error word before the barrier.
__device__ __forceinline__ bool wg_wait(const AgGemmParams& p, const int* f0, int n, int wave, int lane, int q,
                                        int phase, int pos) {
    if (wave == 0) {
        for (int b = 0; b < n; b += 64) {
            const bool mine = b + lane < n;
            const int* f = f0 + (size_t)(mine ? b + lane : b) * kFlagStride;
            const long long t0 = wall_clock64();
            unsigned spins = 0;
            while (__ballot(mine && __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < 1) != 0) {
                __builtin_amdgcn_s_sleep(2);
                if ((++spins & 31u) == 0) {
                    if (__hip_atomic_load(&p.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
                    if (wall_clock64() - t0 > p.spin_limit) {
                        if (lane == 0) report_timeout(p.status, q, phase, pos);
                        break;
                    }
                }
            }
        }
        asm volatile("" ::: "memory");
    }
    lds_barrier();
    return __hip_atomic_load(&p.status->code, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0;
}

// Set flag f once, after every wave's stores are complete (the caller's K
// loop ends with a full wait and a workgroup barrier); with the check_flags
// debug knob its old value must be 0, else RING_EPROTOCOL at (q, g, pos).
__device__ __forceinline__ void wg_signal(const AgGemmParams& p, int* f, int tid, int q, int g, int pos) {
    if (tid == 0) {
        if (p.check_flags) {
            if (__hip_atomic_fetch_add(f, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0)
                report_error(p.status, RING_EPROTOCOL, q, g, pos);
        } else {
            __hip_atomic_fetch_add(f, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <class G, bool GELU>
__device__ void ag_gemm_body(const AgGemmParams& p, unsigned short* lds) {
    constexpr int BN = G::BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / G::WC, wc = wave % G::WC;
    const int P = p.P;
    const int q = blockIdx.x % P;
    const int grp = blockIdx.x / P;
    const int left = (q - 1 + P) % P;
    const int Mc = p.M / P;
    // the workspace's record of data earlier calls left: none may lie under
    // the panel flags (every wave sees the same answer and leaves)
    if (blockIdx.x == 0 && tid == 0) ws_add_data(p.status, p.ws_data);
    if (!ws_ok(p.status, ws_record(p.status), p.ws_zero, lane)) return;

    ForwardHook<G> fw;
    fw.init(lds, lane, wave);
    for (int f = 0; f < P; ++f) {
        const int c = (q - f + P) % P;
        for (int pos = grp; pos < p.tpc; pos += p.groups) {
            const int pr = pos / p.tn, tc = pos % p.tn;
            int k0, k1;
            forward_range(p, tc, k0, k1);
            fw.at(p.Af[q] + ((size_t)c * Mc + (size_t)pr * kBM) * p.K, p.K, lane, wave, k0, k1);
            f32x16 acc[kMI][G::NI];
            if (f < 2) {
                // the local block, then the left rank's, straight from the inputs
                const unsigned short* src = p.As[f == 0 ? q : left];
                gemm_tile_with<G, POL_PLAIN>(p.K, p.N, src, p.B[q], pr, tc, acc, lds, lane, wave, wr, wc, fw);
            } else {
                // the left rank's phase f - 1 tiles of this panel, flagged at
                // consecutive positions.  Those rows reached the device's
                // coherence point (device-scope stores, completed before the
                // flags), and no cache on the way holds an older copy: a
                // launch starts with every L2 invalidated, and in a launch
                // these rows are read only here, in this phase, after the
                // flags.  So the loads may be ordinary ones (measured: the
                // MLP layer 1.5-2.5% faster than with device-scope loads).
                if (!wg_wait(p, ag_flag(p, f - 1, left, pr * p.tn), p.tn, wave, lane, q, f, pos)) return;
                gemm_tile_with<G, POL_PLAIN>(p.K, p.N, p.Af[left], p.B[q], c * p.tm_chunk + pr, tc, acc, lds, lane,
                                             wave, wr, wc, fw);
            }
            // this tile's share of the panel is in A_full[q]: flag it for the
            // right rank's next phase (the last phase has no reader)
            if (f >= 1 && f + 1 < P && !(q == 0 && p.drop_round > 0 && f == p.drop_round))
                wg_signal(p, ag_flag(p, f, q, pos), tid, q, f, pos);
            const size_t at = ((size_t)c * Mc + pr * kBM + wr * kWM) * p.N + tc * BN + wc * G::WN;
            if constexpr (GELU) {
                store_part_rowmajor<G, false, EPI_GELU_BF16>(acc, tile_view(nullptr, 0), (char*)p.C[q] + at * 2,
                                                             p.N, lds, lane, wave);
            } else {
                store_part_rowmajor<G, false, EPI_F32>(acc, tile_view(nullptr, 0), (char*)p.C[q] + at * 4, p.N,
                                                       lds, lane, wave);
            }
        }
    }
}

template <class G, bool GELU>
__global__ __launch_bounds__(64 * G::NW, G::kWGsPerCU) void ag_gemm_kernel(AgGemmParams p) {
    __shared__ __attribute__((aligned(16))) unsigned short lds[G::kLds / 2];
    ag_gemm_body<G, GELU>(p, lds);
    // The last workgroup to finish clears the panel flags for the next call
    // (every reader is done by then; an abandoned launch gets here too).
    // Wave 0 counts the workgroup out and, if it was the last, clears.
    __syncthreads();
    if (threadIdx.x < 64) {
        int prev = 0;
        if (threadIdx.x == 0)
            prev = __hip_atomic_fetch_add(p.done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        prev = __builtin_amdgcn_readfirstlane(prev);
        if (prev == (int)gridDim.x - 1) {
            for (int i = threadIdx.x; i < p.nflags; i += 64)
                __hip_atomic_store(p.flags + (size_t)i * kFlagStride, 0, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if (threadIdx.x == 0) __hip_atomic_store(p.done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- host side
static size_t align256_ag(size_t x) { return (x + 255) / 256 * 256; }

// Sized for 256 x 128 tiles, the narrowest used.
struct AgWs {
    size_t flags_off, flags_bytes, total;
    int nflags;
};

static AgWs ag_ws_layout(int P, size_t MN) {
    AgWs w;
    const size_t tpc = MN / (size_t)P / ((size_t)kBM * 128);
    w.nflags = (int)((size_t)P * P * (tpc ? tpc : 1));
    w.flags_off = kStatusBytes;
    w.flags_bytes = align256_ag((size_t)w.nflags * kFlagStride * sizeof(int));
    w.total = w.flags_off + w.flags_bytes;
    return w;
}

size_t ag_gemm_workspace_bytes(int P, size_t n) {
    if (P < 1 || P > RING_MAX_RANKS || n == 0 || n % ((size_t)P * kBM * 128)) return 0;
    return ag_ws_layout(P, n).total;
}

template <class G, bool GELU>
static int launch_ag_gemm(AgGemmParams& prm, const DevInfo& di, hipStream_t stream) {
    prm.tn = prm.N / G::BN;
    prm.tpc = prm.tm_chunk * prm.tn;
    // at most G::kWGsPerCU workgroups per CU, so on an otherwise idle GPU
    // every workgroup runs at once (tiles wait for the left rank's tiles of
    // the previous phase); the occupancy query confirms the hardware agrees
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, ag_gemm_kernel<G, GELU>, 64 * G::NW, 0) != hipSuccess ||
        occ < G::kWGsPerCU)
        return RING_EHIP;
    long long groups = (long long)di.cus * G::kWGsPerCU / prm.P;
    if (groups > prm.tpc) groups = prm.tpc;
    if (groups < 1) return RING_EUNSUPPORTED;
    prm.groups = (int)groups;
    ag_gemm_kernel<G, GELU><<<dim3((unsigned)(groups * prm.P)), dim3(64 * G::NW), 0, stream>>>(prm);
    return hipGetLastError() == hipSuccess ? RING_OK : RING_EHIP;
}

static bool ag_overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int ag_gemm_run(const void* const* A_shard, const void* const* B, void* const* A_full, void* const* C,
                int P, int M, int N, int K, void* ws, size_t ws_bytes, void* stream, int gelu_bf16,
                WsSpan extra) {
    if (P < 1 || P > RING_MAX_RANKS || M < 0 || N < 0 || K < 0) return RING_EINVAL;
    if (!A_shard || !B || !A_full || !C) return RING_EINVAL;
    if (M == 0 || N == 0) return RING_OK;
    if (M % (kBM * P) || N % 128 || K % 64 || K == 0) return RING_EUNSUPPORTED;
    if (!gemm_views_fit(N, K)) return RING_EUNSUPPORTED;
    const size_t shard_bytes = (size_t)(M / P) * K * 2, full_bytes = (size_t)M * K * 2;
    for (int r = 0; r < P; ++r) {
        if (!A_shard[r] || !B[r] || !A_full[r] || !C[r]) return RING_EINVAL;
        if (((uintptr_t)A_shard[r] | (uintptr_t)B[r] | (uintptr_t)A_full[r] | (uintptr_t)C[r]) & 15)
            return RING_EINVAL;
    }
    // the gathered buffers are written while every shard and gathered buffer
    // is being read: they must not overlap the inputs or each other
    for (int a = 0; a < P; ++a)
        for (int b = 0; b < P; ++b) {
            if (ag_overlap(A_full[a], full_bytes, A_shard[b], shard_bytes)) return RING_EINVAL;
            if (a != b && ag_overlap(A_full[a], full_bytes, A_full[b], full_bytes)) return RING_EINVAL;
        }
    const AgWs lay = ag_ws_layout(P, (size_t)M * N);
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < lay.total) return RING_EWORKSPACE;

    AgGemmParams prm;
    memset(&prm, 0, sizeof prm);
    for (int r = 0; r < P; ++r) {
        prm.As[r] = (const unsigned short*)A_shard[r];
        prm.B[r] = (const unsigned short*)B[r];
        prm.Af[r] = (unsigned short*)A_full[r];
        prm.C[r] = C[r];
    }
    prm.status = (Status*)ws;
    prm.done = (int*)((char*)ws + kDoneOffset);
    prm.flags = (int*)((char*)ws + lay.flags_off);
    prm.nflags = lay.nflags;
    prm.ws_zero = WsSpan{kStatusBytes, lay.flags_off + lay.flags_bytes};
    prm.ws_data = extra;   // the all-gather + GEMM itself leaves no data in the workspace
    const DevInfo di = dev_info();
    const ring_tuning_t tu = tuning();
    prm.check_flags = tu.check_flags;
    prm.spin_limit = (long long)(tu.timeout_s * (double)di.wall_khz * 1000.0);
    prm.drop_round = tu.drop_round;
    prm.P = P;
    prm.M = M;
    prm.N = N;
    prm.K = K;
    prm.tm_chunk = M / P / kBM;
    int bn = tu.gemm_tile_n;
    if (bn == 0) {
        const long long wide_tiles = (long long)prm.tm_chunk * (N / 256);
        bn = (N % 256 == 0 && wide_tiles >= (long long)(di.cus / P)) ? 256 : 128;
    }
    if (bn == 256 && N % 256) return RING_EUNSUPPORTED;
    prm.gelu_bf16 = gelu_bf16 ? 1 : 0;
    const hipStream_t st = (hipStream_t)stream;
    if (prm.gelu_bf16)
        return bn == 256 ? launch_ag_gemm<Geo<256, 8>, true>(prm, di, st) : launch_ag_gemm<Geo<128, 4>, true>(prm, di, st);
    return bn == 256 ? launch_ag_gemm<Geo<256, 8>, false>(prm, di, st) : launch_ag_gemm<Geo<128, 4>, false>(prm, di, st);
}

}  // namespace ringc

extern "C" int all_gather_gemm(const void* const* A_shard, const void* const* B, void* const* A_full,
                               void* const* C, int P, int M, int N, int K, void* ws, size_t ws_bytes,
                               void* stream) {
    return ringc::ag_gemm_run(A_shard, B, A_full, C, P, M, N, K, ws, ws_bytes, stream, 0, ringc::WsSpan{0, 0});
}

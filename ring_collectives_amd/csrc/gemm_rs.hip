// gemm_rs.hip -- GEMM + ring reduce-scatter with tile-level overlap.
//
// Every virtual rank q computes C_q = A_q B_q (bf16 in, fp32 out) and the
// ranks reduce-scatter the products over row-block chunks: chunk c is rows
// [c M/P, (c+1) M/P) and rank q keeps chunk q of sum_q C_q.  The unfused
// meaning is the collective-matmul section of "TPU 与分布式通信原语" (a full
// local matmul, then the ring reduce-scatter of its row blocks); the overlap
// is the "GEMM + ReduceScatter 重叠" pattern of "Triton-distributed 语义": the
// GEMM produces output tiles, signals each one, and the reduce-scatter
// consumes each tile as soon as its signal arrives.
//
// Schedule.  Rank q walks its chunks in the order the ring needs them
// ("全归约 3：Ring——每步大小恒定", Walkthrough: in round s rank q adds its own
// chunk (q - s - 2) mod P to what its left neighbour sends):
//   phase 0      : chunk (q - 1) mod P, the one its right neighbour needs
//                  first; the raw fp32 tile goes to the workspace + flag;
//   phase 1 + s  : chunk (q - s - 2) mod P; the tile is added to the left
//                  neighbour's tile of the previous phase (its raw tile at
//                  s = 0, its partial sum after) and stored + flagged, except
//   phase P - 1  : chunk q itself, whose sum is final and goes to out[q].
// So every rank starts on the tile its neighbour waits for and finishes on
// its own chunk (the threadblock-swizzle idea of "Triton-distributed 语义",
// "线程块交织", turned to the direction of this ring).  The fp32 additions
// are exactly the ring reduce-scatter's: ((C_{c+1} + C_{c+2}) + ...) + C_c.
//
// Tiles.  One workgroup computes one 256 x BN fp32 output tile (256 x 256
// with 8 waves, one workgroup per CU; 256 x 128 with 4 waves, two per CU;
// 256 x 64 with 4 waves, one per CU) with v_mfma_f32_32x32x16_bf16; every
// wave owns a 128 x 64 part (128 x 32 for the narrowest) as 32 x 32 MFMA
// blocks.  K advances through LDS buffers filled by direct global->LDS
// loads one step ahead of the buffers the matrix cores read.  Partial tiles
// travel through the workspace in MFMA fragment order (what one instruction
// of a wave moves is 1 KiB of contiguous memory), and a flag guards each
// wave's part, so producer wave w and consumer wave w of the next rank pair
// up directly.
//
// Work assignment: the work items (phase, position, rank) are numbered phase
// by phase, position by position, the P ranks of a position consecutive, and
// workgroup g of G takes items g, g + G, g + 2G, ...  An item waits only for
// the left rank's item at the same position of the phase before, which has
// a smaller number.  Every workgroup gets to run (G is at most what the CUs
// hold; beside another kernel the rest start as its workgroups finish) and
// works through its items in increasing order, so the smallest unfinished
// item always has its input ready and its workgroup at it: the launch always
// finishes.  Numbering across phases lets a small problem
// (fewer tiles per chunk than workgroup slots) run several phases at once.
#include "gemm_core.h"

#include <hip/hip_runtime.h>
#include <string.h>

namespace ringc {

struct GemmParams {
    const unsigned short* A[RING_MAX_RANKS];   // bf16 M x K, row-major
    const unsigned short* B[RING_MAX_RANKS];   // bf16 K x N, row-major
    void* out[RING_MAX_RANKS];                 // (M / P) x N row-major, fp32 or bf16
    float* work;                               // P x (M x N) fp32, tiles in fragment order
    int* flags;                                // [P-1][P][tpc][4] flags
    Status* status;
    long long spin_limit;
    int P, M, N, K;
    int tm_chunk;                              // tile rows per chunk (M / P / 256)
    int tn;                                    // tile columns (N / BN)
    int tpc;                                   // tiles per chunk
    int batched;                               // P independent products, no reduce-scatter
    int ksplit;                                // batched: K split in this many ranges, each
    float* split;                              //   range's fp32 product at split[(s P + q) M N ..]
    int epi;                                   // what out holds: EPI_F32, EPI_BF16 (the fp32 sum
                                               // rounded once) or EPI_GELU_BF16
    WsSpan ws_zero, ws_data;                   // flags that must start zero; data left behind
    int check_flags;                           // debug: each flag must be 0 when it is set
};

template <class G>
__device__ __forceinline__ int* gflag(const GemmParams& p, int row, int q, int pos, int wave) {
    return p.flags + ((((size_t)row * p.P + q) * p.tpc + pos) * G::NW + wave) * kFlagStride;
}

// One wave's part of tile (tr, tc) of rank q's workspace, fragment order.
template <class G>
__device__ __forceinline__ float* work_part(const GemmParams& p, int q, int tr, int tc, int wave) {
    return p.work + (size_t)q * p.M * p.N + ((size_t)tr * p.tn + tc) * G::kTile +
           (size_t)wave * G::kPart;
}

template <class G>
__global__ __launch_bounds__(64 * G::NW, G::kWGsPerCU) void gemm_rs_kernel(GemmParams p) {
    constexpr int BN = G::BN;
    __shared__ __attribute__((aligned(16))) unsigned short lds[G::kLds / 2];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wave / G::WC, wc = wave % G::WC;
    const int P = p.P;
    // batched: P independent products, no reduce-scatter (each rank's whole
    // product is one chunk, stored straight to out[q]), optionally with K in
    // ksplit ranges whose products go to split (summed by the caller)
    const int S = p.batched ? p.ksplit : 1;
    const int items = p.batched ? P * p.tpc * S : P * P * p.tpc;
    // the workspace's record of data earlier calls left: none may lie under
    // this launch's flags (every wave sees the same answer and leaves)
    if (blockIdx.x == 0 && tid == 0) ws_add_data(p.status, p.ws_data);
    if (!ws_ok(p.status, ws_record(p.status), p.ws_zero, lane)) return;

    for (int it = blockIdx.x; it < items; it += gridDim.x) {
        const int phase = p.batched ? 0 : it / (P * p.tpc);
        const int ks = p.batched ? it / (P * p.tpc) : 0;   // K range of a batched item
        const int pos = (it / P) % p.tpc;
        const int q = it % P;
        const int left = (q - 1 + P) % P;
        const unsigned short* A = p.A[q];
        const unsigned short* B = p.B[q];
        // chunk of this phase (see the schedule above); P = 1 has one phase
        const int c = (P == 1 || p.batched) ? 0
                                            : (phase == 0 ? (q - 1 + P) % P : (q - phase - 1 + 2 * P) % P);
        const bool final_phase = p.batched || (phase == P - 1);
        {
            const int tr = c * p.tm_chunk + pos / p.tn;
            const int tc = pos % p.tn;
            f32x16 acc[kMI][G::NI];
            gemm_tile<G>(p.K, p.N, A, B, tr, tc, acc, lds, lane, wave, wr, wc, ks * (p.K / S), p.K / S);

            // Epilogue.  Each row of 32 x 32 blocks is loaded, added and stored
            // in one go so only a few accumulators are live outside the
            // AGPRs.  The per-lane offsets are recomputed here (the empty asm
            // hides them from loop-invariant hoisting, which would otherwise
            // keep every element address alive across the tile loop).
            unsigned lane16 = (unsigned)lane * 16u;
            asm volatile("" : "+v"(lane16));
            rsrc_t rv = tile_view(nullptr, 0);
            if (phase > 0) {
                // the left neighbour's tile of the previous phase (raw at s = 0)
                int* f = gflag<G>(p, phase - 1, left, pos, wave);
                const int seen = peek_flag(f);
                if (!wait_flag(f, p.status, p.spin_limit, q, phase, pos, lane, seen)) return;
                rv = tile_view(work_part<G>(p, left, tr, tc, wave), G::kPart * 4);
            }
            if (!final_phase) {
                const rsrc_t wv = tile_view(work_part<G>(p, q, tr, tc, wave), G::kPart * 4);
#pragma unroll
                for (int mi = 0; mi < kMI; ++mi) {
                    u32x4 x[G::NI][4];
                    if (phase > 0) {
#pragma unroll
                        for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
                            for (int part = 0; part < 4; ++part)
                                // the neighbour's partial, read once: device scope, streamed
                                x[ni][part] = ld16s<POL_DEV | POL_NT>(rv, lane16, frag_soff<G>(mi, ni, part));
                    }
#pragma unroll
                    for (int ni = 0; ni < G::NI; ++ni) {
                        // one vector base per block; the parts sit 1 KiB apart
                        // and go into the instruction's immediate offset
                        const unsigned vo = lane16 + frag_soff<G>(mi, ni, 0);
#pragma unroll
                        for (int part = 0; part < 4; ++part) {
                            u32x4 o;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float cv = acc[mi][ni][part * 4 + e];
                                o[e] = __float_as_uint(phase > 0 ? __uint_as_float(x[ni][part][e]) + cv : cv);
                            }
                            st16<POL_DEV>(o, wv, vo + (unsigned)part * 1024u);
                        }
                    }
                }
                signal_flag(gflag<G>(p, phase, q, pos, wave), lane, p.check_flags, p.status, q, phase + 1, pos);
            } else {
                // Final sum of chunk q, row-major into out[q]: fp32, rounded
                // once to bf16, or bf16(gelu(bf16(sum))).
                const int lrow0 = (tr - c * p.tm_chunk) * kBM + wr * kWM;   // c == q unless batched
                const size_t at = (size_t)lrow0 * p.N + tc * BN + wc * G::WN;
                if (S > 1) {
                    char* ob = (char*)(p.split + (size_t)(ks * P + q) * p.M * p.N) + at * 4;
                    store_part_rowmajor<G, false, EPI_F32>(acc, rv, ob, p.N, lds, lane, wave);
                } else if (p.epi == EPI_BF16) {
                    char* ob = (char*)p.out[q] + at * 2;
                    if (phase > 0) store_part_rowmajor<G, true, EPI_BF16>(acc, rv, ob, p.N, lds, lane, wave);
                    else store_part_rowmajor<G, false, EPI_BF16>(acc, rv, ob, p.N, lds, lane, wave);
                } else if (p.epi == EPI_GELU_BF16) {
                    char* ob = (char*)p.out[q] + at * 2;
                    if (phase > 0) store_part_rowmajor<G, true, EPI_GELU_BF16>(acc, rv, ob, p.N, lds, lane, wave);
                    else store_part_rowmajor<G, false, EPI_GELU_BF16>(acc, rv, ob, p.N, lds, lane, wave);
                } else {
                    char* ob = (char*)p.out[q] + at * 4;
                    if (phase > 0) store_part_rowmajor<G, true, EPI_F32>(acc, rv, ob, p.N, lds, lane, wave);
                    else store_part_rowmajor<G, false, EPI_F32>(acc, rv, ob, p.N, lds, lane, wave);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- host side
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Shapes come in multiples of 256 x 128 (kShapeFloats); tiles are never
// narrower than 64 columns, so the flag table is sized for 256 x 64 tiles
// whatever width a call uses.
constexpr size_t kShapeFloats = (size_t)kBM * 128;
constexpr size_t kMinTileFloats = (size_t)kBM * 64;

struct GemmWs {
    size_t flags_off, flags_bytes, work_off, work_bytes, total;
};

static GemmWs gemm_ws_layout(int P, size_t MN) {
    GemmWs w;
    const size_t tpc = MN / (size_t)P / kMinTileFloats;
    const size_t rows = P > 1 ? (size_t)(P - 1) : 1;
    w.flags_off = kStatusBytes;
    w.flags_bytes = align256(rows * (size_t)P * (tpc ? tpc : 1) * 4 * kFlagStride * sizeof(int));
    w.work_off = w.flags_off + w.flags_bytes;
    w.work_bytes = P > 1 ? align256((size_t)P * MN * sizeof(float)) : 0;
    w.total = w.work_off + w.work_bytes;
    return w;
}

size_t gemm_rs_workspace_bytes(int P, size_t n) {
    if (P < 1 || P > RING_MAX_RANKS || n == 0 || n % ((size_t)P * kShapeFloats)) return 0;
    return gemm_ws_layout(P, n).total;
}

template <class G>
static int launch_gemm_rs(GemmParams& prm, const DevInfo& di, hipStream_t stream) {
    prm.tn = prm.N / G::BN;
    prm.tpc = prm.tm_chunk * prm.tn;
    // at most G::kWGsPerCU workgroups per CU, so on an otherwise idle GPU
    // every workgroup runs at once; the occupancy query confirms the
    // hardware agrees
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_rs_kernel<G>, 64 * G::NW, 0) != hipSuccess ||
        occ < G::kWGsPerCU)
        return RING_EHIP;
    long long grid = (long long)di.cus * G::kWGsPerCU;
    const long long items = (long long)prm.P * (prm.batched ? prm.ksplit : prm.P) * prm.tpc;
    if (grid > items) grid = items;
    hipLaunchKernelGGL(gemm_rs_kernel<G>, dim3((unsigned)grid), dim3(64 * G::NW), 0, stream, prm);
    return hipGetLastError() == hipSuccess ? RING_OK : RING_EHIP;
}

// The status word sits at ws; the flag table and the partial tiles start
// region_off bytes later than in a call of its own (the MLP layer puts them
// behind the all-gather's flags).
int gemm_rs_run(const void* const* A, const void* const* B, void* const* out, int P, int M, int N, int K,
                void* ws, size_t ws_bytes, void* stream, int epi, size_t region_off, int batched, int ksplit,
                float* split, WsSpan extra) {
    if (P < 1 || P > RING_MAX_RANKS || M < 0 || N < 0 || K < 0) return RING_EINVAL;
    if (!A || !B || !out) return RING_EINVAL;
    if (M == 0 || N == 0) return RING_OK;
    const int chunks = batched ? 1 : P;   // row blocks each rank's product splits into
    if (M % (kBM * chunks) || N % 128 || K % 64 || K == 0) return RING_EUNSUPPORTED;
    if (!gemm_views_fit(N, K)) return RING_EUNSUPPORTED;
    if (ksplit < 1 || (ksplit > 1 && (!batched || !split || epi != EPI_F32 || K % (64 * ksplit))))
        return RING_EINVAL;
    for (int r = 0; r < P; ++r) {
        if (!A[r] || !B[r] || !out[r]) return RING_EINVAL;
        if (((uintptr_t)A[r] | (uintptr_t)B[r] | (uintptr_t)out[r]) & 15) return RING_EINVAL;
    }
    const size_t MN = (size_t)M * N;
    GemmWs lay = gemm_ws_layout(batched ? 1 : P, MN);
    lay.flags_off += region_off;
    lay.work_off += region_off;
    lay.total += region_off;
    if (!ws || ((uintptr_t)ws & 255) || (region_off & 255) || ws_bytes < lay.total) return RING_EWORKSPACE;

    GemmParams prm;
    memset(&prm, 0, sizeof prm);
    for (int r = 0; r < P; ++r) {
        prm.A[r] = (const unsigned short*)A[r];
        prm.B[r] = (const unsigned short*)B[r];
        prm.out[r] = out[r];
    }
    prm.work = (float*)((char*)ws + lay.work_off);
    prm.flags = (int*)((char*)ws + lay.flags_off);
    prm.status = (Status*)ws;
    // batched products use no flags; the reduce-scatter's partial tiles stay
    // in the workspace
    prm.ws_zero = batched ? WsSpan{0, 0} : WsSpan{kStatusBytes, lay.flags_off + lay.flags_bytes};
    WsSpan data = lay.work_bytes && !batched ? WsSpan{lay.work_off, lay.work_off + lay.work_bytes} : WsSpan{0, 0};
    if (extra.hi > extra.lo) {
        if (data.hi <= data.lo) data = extra;
        else data = WsSpan{data.lo < extra.lo ? data.lo : extra.lo, data.hi > extra.hi ? data.hi : extra.hi};
    }
    prm.ws_data = data;
    const DevInfo di = dev_info();
    const ring_tuning_t tu = tuning();
    prm.check_flags = tu.check_flags;
    prm.spin_limit = (long long)(tu.timeout_s * (double)di.wall_khz * 1000.0);
    prm.P = P;
    prm.M = M;
    prm.N = N;
    prm.K = K;
    prm.tm_chunk = M / chunks / kBM;
    prm.batched = batched ? 1 : 0;
    prm.ksplit = ksplit;
    prm.split = split;
    int bn = tu.gemm_tile_n;
    if (bn == 0) {
        // Wide tiles need less operand traffic per flop but make half as
        // many work items; they pay off once there is at least one wide
        // item per CU (the items of all phases count: phases overlap).
        // When even the 64-wide items number at most one per CU, those
        // spread the work over more CUs.  A CU holds one 64-wide workgroup,
        // so with more of them some CUs would run two in turn, and the
        // 128-wide tiles, two workgroups per CU at once, are faster.
        const long long items128 = (long long)P * (batched ? ksplit : P) * prm.tm_chunk * (N / 128);
        const long long cus = di.cus;
        bn = (N % 256 == 0 && items128 / 2 >= cus) ? 256 : 2 * items128 <= cus ? 64 : 128;
    }
    if (bn == 256 && N % 256) return RING_EUNSUPPORTED;
    if (epi != EPI_F32 && epi != EPI_BF16 && epi != EPI_GELU_BF16) return RING_EINVAL;
    prm.epi = epi;
    const hipStream_t st = (hipStream_t)stream;
    return bn == 256 ? launch_gemm_rs<Geo<256, 8>>(prm, di, st)
                     : bn == 128 ? launch_gemm_rs<Geo<128, 4>>(prm, di, st) : launch_gemm_rs<Geo<64, 4>>(prm, di, st);
}

}  // namespace ringc

extern "C" int gemm_reduce_scatter(const void* const* A, const void* const* B, void* const* out,
                                   int P, int M, int N, int K, void* ws, size_t ws_bytes,
                                   void* stream) {
    return ringc::gemm_rs_run(A, B, out, P, M, N, K, ws, ws_bytes, stream, ringc::EPI_F32, 0, 0, 1, nullptr,
                              ringc::WsSpan{0, 0});
}

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
// with 8 waves, one workgroup per CU, or 256 x 128 with 4 waves, two per CU)
// with v_mfma_f32_32x32x16_bf16; every wave owns a 128 x 64 part as 32 x 32
// MFMA blocks.  K advances through LDS buffers filled by direct global->LDS
// loads one step ahead of the buffers the matrix cores read.  Partial tiles
// travel through the workspace in MFMA fragment order (what one instruction
// of a wave moves is 1 KiB of contiguous memory), and a flag guards each
// wave's part, so producer wave w and consumer wave w of the next rank pair
// up directly.
//
// Work assignment: workgroup g serves rank g % P and tile positions
// g / P, g / P + G / P, ... of every chunk, phase by phase.  A tile of phase
// f waits only for the left rank's tile at the same position of phase f-1,
// held by the neighbouring workgroup and earlier in its order, and the P
// workgroups of a ring are consecutive, so resident rings always finish.
#include "ring_device.h"

#include <hip/hip_runtime.h>
#include <string.h>

namespace ringc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kBM = 256;      // output tile rows
constexpr int kWM = 128;      // rows of a wave's part of the tile
constexpr int kMI = kWM / 32; // 32 x 32 MFMA blocks down a wave's part

// Tile geometry for an output tile of kBM x BN computed by NW waves, arranged
// 2 down x NW / 2 across: wave w owns rows (w / WC) * 128 .. +127 and columns
// (w % WC) * WN .. + WN - 1, a part of 128 x 64 (4 x 2 MFMA blocks of 32 x 32,
// 128 accumulator registers, so two waves fit on a SIMD).
//   BN = 256, NW = 8: one workgroup per CU; a compute step covers 64 of K;
//   BN = 128, NW = 4: two workgroups per CU; a step covers 32 of K.
// Both run two waves per SIMD, so one wave's LDS reads and waits overlap the
// other's matrix-core work.  The wide tile needs a third less operand traffic
// per flop and wins once there are enough tiles to fill the CUs.
// A is staged 64 deep in K whatever the step, so every A row of a stage is one
// whole 128-byte line: rows of 64 bytes cost about twice the fabric requests
// per byte (each load instruction touches 16 half-used lines instead of 8
// full ones).  With BN = 128 an A stage therefore serves two steps.  Two A
// and two B buffers: 128 KiB for BN = 256, 80 KiB (twice per CU) for 128.
template <int BN_, int NW_> struct Geo {
    static constexpr int BN = BN_;                       // output tile columns
    static constexpr int NW = NW_;                       // waves per workgroup
    static constexpr int WC = NW / 2;                    // waves across the tile
    static constexpr int BKA = 64;                       // K per A stage
    static constexpr int BKB = BN == 256 ? 64 : 32;      // K per B stage = per step
    static constexpr int R = BKA / BKB;                  // steps per A stage
    static constexpr int KK = BKB / 16;                  // MFMA k-steps per step
    static constexpr int WN = BN / WC;                   // columns of a wave's part
    static constexpr int NI = WN / 32;                   // 32 x 32 blocks across it
    static constexpr int kStageA = kBM * BKA * 2;        // bytes of one A buffer
    static constexpr int kStageB = BKB * BN * 2;         // bytes of one B buffer
    static constexpr int kBBase = 2 * kStageA;           // B buffers follow the two A buffers
    static constexpr int kLds = 2 * kStageA + 2 * kStageB;
    static constexpr int kARowBytes = BKA * 2;           // 128
    static constexpr int kAC = BKA / 8;                  // 16-byte chunks per A row
    static constexpr int kARows = 64 / kAC;              // A rows per 1-KiB load
    static constexpr int kLoadsA = kBM / kARows / NW;    // per wave per A stage
    static constexpr int kBRowBytes = BN * 2;
    static constexpr int kBRows = 1024 / kBRowBytes;     // B rows per 1-KiB load
    static constexpr int kLoadsB = BKB / kBRows / NW;    // per wave per B stage
    static constexpr int kPart = kWM * WN;               // floats of a wave's part
    static constexpr int kTile = kBM * BN;
    static constexpr int kEpiStride = WN + 4;            // LDS floats per row of the final transpose
    static constexpr int kEpiWave = 32 * kEpiStride;     // a wave's 32-row band
    static constexpr int kWGsPerCU = BN == 256 ? 1 : 2;
    // XOR applied to the 16-byte chunk index of A row m in LDS
    static __device__ __forceinline__ int swz_a(int m) { return (m >> 1) & 7; }
    static_assert(kLds * kWGsPerCU <= 160 * 1024, "LDS");
    static_assert(NW * kEpiWave * 4 <= kLds, "epilogue LDS");
    static_assert(kBM % (NW * kARows) == 0 && BKB % (NW * kBRows) == 0, "load split");
};

struct GemmParams {
    const unsigned short* A[RING_MAX_RANKS];   // bf16 M x K, row-major
    const unsigned short* B[RING_MAX_RANKS];   // bf16 K x N, row-major
    float* out[RING_MAX_RANKS];                // fp32 (M / P) x N, row-major
    float* work;                               // P x (M x N) fp32, tiles in fragment order
    int* flags;                                // [P-1][P][tpc][4] flags
    Status* status;
    long long spin_limit;
    int P, M, N, K;
    int tm_chunk;                              // tile rows per chunk (M / P / 256)
    int tn;                                    // tile columns (N / BN)
    int tpc;                                   // tiles per chunk
    int groups;                                // rings of workgroups (gridDim.x / P)
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

// Fragment order of a wave's part: the part-th 4 accumulators of block (mi, ni)
// of lane l sit at byte lane * 16 + frag_soff(mi, ni, part), so one
// instruction of a wave moves 1 KiB of contiguous memory.
template <class G>
__device__ __forceinline__ unsigned frag_soff(int mi, int ni, int part) {
    return (unsigned)(((mi * G::NI + ni) * 4 + part) * 1024);
}

// LDS layout (bytes): A buffers at 0 and kStageA (256 rows m x 64 k, 128
// bytes per row), B buffers at kBBase and kBBase + kStageB (BKB rows k x BN
// n); no padding.  All are filled by direct global->LDS loads (one
// instruction = 64 lanes x 16 B = 1 KiB of consecutive LDS) and spread over
// the banks by XOR-ing the 16-byte chunk index:
//   A: chunk c of row m is stored at chunk c ^ ((m >> 1) & 7)
//   B: chunk c of row k is stored at chunk c ^ (4 (k & 3))
// The LDS has 64 banks of 4 bytes and serves 16 lanes of a 16-byte read, or
// 32 lanes of an 8-byte read, per cycle; with these swizzles the 16 rows of an
// A fragment read, and the 4 rows x 2 column groups of a transposed B read,
// land on 256 distinct bytes, so neither read has a bank conflict.
__device__ __forceinline__ lds_void* lds_at(unsigned short* lds, unsigned byte) {
    return (lds_void*)((__attribute__((address_space(3))) char*)(lds_void*)lds + byte);
}

// Workgroup barrier for the LDS stages only.  __syncthreads() also fences
// global memory, for which the compiler drains every outstanding load first
// (s_waitcnt vmcnt(0)), prefetched stages included, which would serialise the
// pipeline.  The direct loads into LDS are waited for explicitly (wait_vm),
// so the barrier only has to order this wave's LDS reads (lgkmcnt(0)) and
// keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most `n` of this wave's vector memory operations are in flight.
__device__ __forceinline__ void wait_vm(int n) {
    if (n >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (n >= 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (n >= 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// C tile (tr, tc) of A_q B_q into acc (the wave's part).
//
// MFMA operands (v_mfma_f32_32x32x16_bf16): lane l holds A[m = l % 32][k =
// 8 (l / 32) + t] and B[k = 8 (l / 32) + t][n = l % 32], t = 0..7.  A is read
// with ds_read_b128 (8 consecutive k of one row).  B comes from its natural
// k-major layout through the LDS transpose read ds_read_b64_tr_b16: within
// each group of 16 lanes, when lane j points at row kb + j / 4, columns
// cb + 4 (j % 4) .. +3, lane i receives rows kb .. kb+3 of column cb + i, so
// two such reads give a lane its 8 consecutive k of one column.
template <class G>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, const unsigned short* __restrict__ A,
                                          const unsigned short* __restrict__ B, int tr, int tc,
                                          f32x16 (&acc)[kMI][G::NI], unsigned short* lds,
                                          int lane, int wave, int wr, int wc) {
    constexpr int BN = G::BN;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

    const int K = p.K, N = p.N;
    // A panel: 256 rows x K; B panel: K rows x BN columns (row stride N).
    const rsrc_t Av = tile_view(A + (size_t)tr * kBM * K, (long long)kBM * K * 2);
    const rsrc_t Bv = tile_view(B + (size_t)tc * BN, ((long long)(K - 1) * N + BN) * 2);

    // Direct loads.  A instruction i of wave w fills rows 8 (kLoadsA w + i)
    // .. +7 (lane: row + lane / 8, stored chunk lane % 8); B instruction i
    // fills kBRows rows of k (lane: row + lane / (BN / 8), stored chunk
    // lane % (BN / 8)).  Each lane fetches the logical chunk its stored
    // position holds.  Both swizzles depend on the lane and on the parity of
    // the instruction index (the first row of an A load is a multiple of 8;
    // of a B load, a multiple of kBRows).
    unsigned a_voff[2], b_voff[2];
    constexpr int BC = BN / 8;                             // chunks per B row
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int m = par * G::kARows + lane / G::kAC;     // row mod 16 of this lane
        a_voff[par] = (unsigned)(((lane / G::kAC) * K + ((lane % G::kAC) ^ G::swz_a(m)) * 8) * 2);
        const int kr = par * G::kBRows + lane / BC;        // row mod 4 of this lane
        const int cb = (lane % BC) ^ (4 * (kr & 3));
        b_voff[par] = (unsigned)(((lane / BC) * N + cb * 8) * 2);
    }
    auto issue_a = [&](int st, int slot) {                 // A stage st (K 64 st ..)
        const unsigned base = (unsigned)(slot * G::kStageA);
#pragma unroll
        for (int i = 0; i < G::kLoadsA; ++i) {
            const int r0 = (wave * G::kLoadsA + i) * G::kARows;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(Av, lds_at(lds, base + r0 * G::kARowBytes), 16,
                                                     a_voff[i & 1],
                                                     (unsigned)((r0 * K + st * G::BKA) * 2), 0, POL_PLAIN);
        }
    };
    auto issue_b = [&](int st, int slot) {                 // B stage st (K BKB st ..)
        const unsigned base = (unsigned)(G::kBBase + slot * G::kStageB);
#pragma unroll
        for (int i = 0; i < G::kLoadsB; ++i) {
            const int k0 = (wave * G::kLoadsB + i) * G::kBRows;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(Bv, lds_at(lds, base + k0 * G::kBRowBytes), 16,
                                                     b_voff[i & 1],
                                                     (unsigned)((st * G::BKB + k0) * N * 2), 0, POL_PLAIN);
        }
    };

    // Fragment read offsets (bytes within a buffer).
    //   A (mi, ka): row wr*128 + mi*32 + l%32, chunk (2 ka + l/32) ^ swz_a(l % 32),
    //     ka = the 16-wide k-step within the A stage
    //   B (ni, kk, half h): row kk*16 + 8 (g/2) + 4h + i/4, column
    //     wc*WN + ni*32 + 16 (g%2) + 4 (i%4), g = l/16, i = l%16
    unsigned a_off[G::BKA / 16], b_off[G::NI];
#pragma unroll
    for (int ka = 0; ka < G::BKA / 16; ++ka)
        a_off[ka] = (unsigned)((wr * kWM + (lane & 31)) * G::kARowBytes +
                               (((2 * ka + (lane >> 5)) ^ G::swz_a(lane & 31)) * 16));
    {
        const int g = lane >> 4, i = lane & 15;
        const int krow = 8 * (g >> 1) + (i >> 2);
#pragma unroll
        for (int ni = 0; ni < G::NI; ++ni) {
            const int n = wc * G::WN + ni * 32 + 16 * (g & 1) + 4 * (i & 3);
            const int chunk = (n >> 3) ^ (4 * (krow & 3));
            b_off[ni] = (unsigned)(krow * G::kBRowBytes + chunk * 16 + (n & 7) * 2);
        }
    }
    auto read_frags = [&](unsigned abase, int ka, unsigned bbase, int kk, bf16x8 (&af)[kMI],
                          bf16x8 (&bf)[G::NI]) {
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi)
            af[mi] = *(const bf16x8*)((const char*)lds + abase + a_off[ka] + mi * 32 * G::kARowBytes);
#pragma unroll
        for (int ni = 0; ni < G::NI; ++ni) {
            const unsigned o = bbase + b_off[ni] + kk * 16 * G::kBRowBytes;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_at(lds, o));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)lds_at(lds, o + 4 * G::kBRowBytes));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            bf[ni] = __builtin_bit_cast(bf16x8, v);
        }
    };

    // Pipeline, in steps of BKB of K: A stage p serves steps R p .. R p + R - 1.
    // At the start of step t (after the barrier, so every wave is done with
    // step t - 1) the workgroup issues B stage t + 1 into the buffer step t - 1
    // used and, on the first step of an A stage, A stage p + 1 into the
    // buffer A stage p - 1 used.  B goes first, so at the top of the next
    // step this wave can wait for its B loads and leave the A loads of the
    // stage after in flight (R = 2, odd steps).  Past the end of K the issues
    // re-read the last stage into the free buffer (never read again).
    const int KT = K / G::BKB;                 // steps
    const int KA = K / G::BKA;                 // A stages
    __syncthreads();   // the previous tile's epilogue may still be reading LDS
    issue_b(0, 0);
    issue_a(0, 0);
    for (int p = 0; p < KA; ++p) {
#pragma unroll
        for (int r = 0; r < G::R; ++r) {
            const int t = p * G::R + r;
            if (r == 0) wait_vm(0);                // B stage t and A stage p have landed
            else wait_vm(G::kLoadsA);              // B stage t has; A stage p + 1 may be in flight
            lds_barrier();                         // everyone's has; buffers of step t - 1 are free
            issue_b(t + 1 < KT ? t + 1 : KT - 1, (t + 1) & 1);
            if (r == 0) issue_a(p + 1 < KA ? p + 1 : KA - 1, (p + 1) & 1);
            const unsigned abase = (unsigned)((p & 1) * G::kStageA);
            const unsigned bbase = (unsigned)(G::kBBase + (t & 1) * G::kStageB);
            // The reads of k-step kk + 1 are issued before the MFMAs of k-step
            // kk, each MFMA waiting only for the reads it consumes.  The
            // scheduling fences hold that order; left alone, the compiler pairs
            // each read with its use through one register set and exposes the
            // LDS latency once per block.
            bf16x8 af[2][kMI], bf[2][G::NI];
            read_frags(abase, r * G::KK, bbase, 0, af[0], bf[0]);
#pragma unroll
            for (int kk = 0; kk < G::KK; ++kk) {
                if (kk + 1 < G::KK)
                    read_frags(abase, r * G::KK + kk + 1, bbase, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < G::NI; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            af[kk & 1][mi], bf[kk & 1][ni], acc[mi][ni], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    wait_vm(0);        // the trailing loads have landed
    __syncthreads();   // all waves are done with the stages before the epilogue uses LDS
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
    const int q = blockIdx.x % P;
    const int grp = blockIdx.x / P;
    const int left = (q - 1 + P) % P;
    const unsigned short* A = p.A[q];
    const unsigned short* B = p.B[q];

    for (int phase = 0; phase < P; ++phase) {
        // chunk of this phase (see the schedule above); P = 1 has one phase
        const int c = P == 1 ? 0 : (phase == 0 ? (q - 1 + P) % P : (q - phase - 1 + 2 * P) % P);
        const bool final_phase = (phase == P - 1);
        for (int pos = grp; pos < p.tpc; pos += p.groups) {
            const int tr = c * p.tm_chunk + pos / p.tn;
            const int tc = pos % p.tn;
            f32x16 acc[kMI][G::NI];
            gemm_tile<G>(p, A, B, tr, tc, acc, lds, lane, wave, wr, wc);

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
                                x[ni][part] = ld16s<POL_DEV>(rv, lane16, frag_soff<G>(mi, ni, part));
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
                signal_flag(gflag<G>(p, phase, q, pos, wave), lane);
            } else {
                // Final sum of chunk q, row-major into out[q].  Each wave turns
                // its part around in its own slice of LDS (free after the K
                // loop), 32 rows at a time, and writes whole row segments.
                int lds_lane = wave * G::kEpiWave + 4 * (lane >> 5) * G::kEpiStride + (lane & 31);
                asm volatile("" : "+v"(lds_lane));
                float* stage_lane = reinterpret_cast<float*>(lds) + lds_lane;   // scatter base
                constexpr int VPR = G::WN / 4;                                  // 16-byte vectors per row
                constexpr int RPS = 64 / VPR;                                   // rows per gather step
                int lds_row = wave * G::kEpiWave + (lane / VPR) * G::kEpiStride + (lane % VPR) * 4;
                asm volatile("" : "+v"(lds_row));
                const float* gather_lane = reinterpret_cast<const float*>(lds) + lds_row;
                const int lrow0 = (tr - q * p.tm_chunk) * kBM + wr * kWM;
                float* ob = p.out[q] + (size_t)lrow0 * p.N + tc * BN + wc * G::WN;
                const rsrc_t ov = tile_view(ob, ((long long)(kWM - 1) * p.N + G::WN) * 4);
                unsigned lane_out = (unsigned)(((lane / VPR) * p.N + (lane % VPR) * 4) * 4);
                asm volatile("" : "+v"(lane_out));
#pragma unroll
                for (int mi = 0; mi < kMI; ++mi) {
                    u32x4 x[G::NI][4];
                    if (phase > 0) {
#pragma unroll
                        for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
                            for (int part = 0; part < 4; ++part)
                                x[ni][part] = ld16s<POL_DEV>(rv, lane16, frag_soff<G>(mi, ni, part));
                    }
#pragma unroll
                    for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const float cv = acc[mi][ni][v];
                            const float o = phase > 0 ? __uint_as_float(x[ni][v >> 2][v & 3]) + cv : cv;
                            stage_lane[(8 * (v >> 2) + (v & 3)) * G::kEpiStride + ni * 32] = o;
                        }
                    // 32 rows x WN columns: in step i lane l reads 16 bytes of
                    // row RPS i + l / VPR at column 4 (l % VPR)
#pragma unroll
                    for (int i = 0; i < 32 / RPS; ++i) {
                        const u32x4 o = *(const u32x4*)(gather_lane + RPS * i * G::kEpiStride);
                        st16<POL_PLAIN>(o, ov, lane_out + (unsigned)(((mi * 32 + RPS * i) * p.N) * 4));
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------- host side
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Tiles are never narrower than 128 columns, so the flag table is sized for
// 256 x 128 tiles whatever width a call uses.
constexpr size_t kMinTileFloats = (size_t)kBM * 128;

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
    if (P < 1 || P > RING_MAX_RANKS || n == 0 || n % ((size_t)P * kMinTileFloats)) return 0;
    return gemm_ws_layout(P, n).total;
}

template <class G>
static int launch_gemm_rs(GemmParams& prm, const DevInfo& di, hipStream_t stream) {
    prm.tn = prm.N / G::BN;
    prm.tpc = prm.tm_chunk * prm.tn;
    // at most G::kWGsPerCU workgroups per CU, so every ring of P workgroups is
    // resident; the occupancy query confirms the hardware agrees
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_rs_kernel<G>, 64 * G::NW, 0) != hipSuccess ||
        occ < G::kWGsPerCU)
        return RING_EHIP;
    long long groups = (long long)di.cus * G::kWGsPerCU / prm.P;
    if (groups > prm.tpc) groups = prm.tpc;
    if (groups < 1) return RING_EUNSUPPORTED;   // more ranks than workgroup slots
    prm.groups = (int)groups;
    hipLaunchKernelGGL(gemm_rs_kernel<G>, dim3((unsigned)(groups * prm.P)), dim3(64 * G::NW), 0, stream, prm);
    return hipGetLastError() == hipSuccess ? RING_OK : RING_EHIP;
}

}  // namespace ringc

using namespace ringc;

extern "C" int gemm_reduce_scatter(const void* const* A, const void* const* B, void* const* out,
                                   int P, int M, int N, int K, void* ws, size_t ws_bytes,
                                   void* stream) {
    if (P < 1 || P > RING_MAX_RANKS || M < 0 || N < 0 || K < 0) return RING_EINVAL;
    if (!A || !B || !out) return RING_EINVAL;
    if (M == 0 || N == 0) return RING_OK;
    if (M % (kBM * P) || N % 128 || K % 64 || K == 0) return RING_EUNSUPPORTED;
    for (int r = 0; r < P; ++r) {
        if (!A[r] || !B[r] || !out[r]) return RING_EINVAL;
        if (((uintptr_t)A[r] | (uintptr_t)B[r] | (uintptr_t)out[r]) & 15) return RING_EINVAL;
    }
    const size_t MN = (size_t)M * N;
    const GemmWs lay = gemm_ws_layout(P, MN);
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < lay.total) return RING_EWORKSPACE;

    GemmParams prm;
    memset(&prm, 0, sizeof prm);
    for (int r = 0; r < P; ++r) {
        prm.A[r] = (const unsigned short*)A[r];
        prm.B[r] = (const unsigned short*)B[r];
        prm.out[r] = (float*)out[r];
    }
    prm.work = (float*)((char*)ws + lay.work_off);
    prm.flags = (int*)((char*)ws + lay.flags_off);
    prm.status = (Status*)ws;
    const DevInfo di = dev_info();
    const ring_tuning_t tu = tuning();
    prm.spin_limit = (long long)(tu.timeout_s * (double)di.wall_khz * 1000.0);
    prm.P = P;
    prm.M = M;
    prm.N = N;
    prm.K = K;
    prm.tm_chunk = M / P / kBM;
    int bn = tu.gemm_tile_n;
    if (bn == 0) {
        // Wide tiles need less operand traffic per flop but make half as
        // many workgroups; they pay off once every CU gets at least one wide
        // tile per chunk.
        const long long wide_tiles = (long long)prm.tm_chunk * (N / 256);
        bn = (N % 256 == 0 && wide_tiles >= (long long)(di.cus / P)) ? 256 : 128;
    }
    if (bn == 256 && N % 256) return RING_EUNSUPPORTED;
    return bn == 256 ? launch_gemm_rs<Geo<256, 8>>(prm, di, (hipStream_t)stream)
                     : launch_gemm_rs<Geo<128, 4>>(prm, di, (hipStream_t)stream);
}

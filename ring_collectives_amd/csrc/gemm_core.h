// gemm_core.h -- the MFMA GEMM tile shared by the fused GEMM + reduce-scatter
// and all-gather + GEMM kernels: tile geometry, the direct global->LDS load
// pipeline, fragment reads for v_mfma_f32_32x32x16_bf16, and the row-major
// store of a finished tile.
#pragma once

#include "ring_device.h"

#include <hip/hip_runtime.h>

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
// 128 accumulator registers, so two waves fit on a SIMD) or, for BN = 64,
// 128 x 32.
//   BN = 256, NW = 8: one workgroup per CU; a compute step covers 64 of K;
//   BN = 128, NW = 4: two workgroups per CU; a step covers 32 of K;
//   BN = 64,  NW = 4: one workgroup per CU, four stages deep; a step covers
//                     64 of K.
// With enough tiles the first two run two waves per SIMD, so one wave's LDS
// reads and waits overlap the other's matrix-core work.  The wide tile needs
// a third less operand traffic per flop and wins once there are enough tiles
// to fill the CUs; the narrow one is for products with too few 128-wide tiles
// to give every CU one (a few hundred tokens), where it halves each tile's
// work.  There a CU holds one workgroup with one wave per SIMD and nothing
// else to run while a stage loads, so the narrow tile keeps three stages in
// flight instead of one: with one, every step waited out a whole load
// latency.
// A is staged 64 deep in K whatever the step, so every A row of a stage is one
// whole 128-byte line: rows of 64 bytes cost about twice the fabric requests
// per byte (each load instruction touches 16 half-used lines instead of 8
// full ones).  With BN = 128 an A stage therefore serves two steps.  NS A and
// NS B buffers: 128 KiB for BN = 256, 80 KiB (twice per CU) for 128, 160 KiB
// for 64.
template <int BN_, int NW_> struct Geo {
    static constexpr int BN = BN_;                       // output tile columns
    static constexpr int NW = NW_;                       // waves per workgroup
    static constexpr int WC = NW / 2;                    // waves across the tile
    static constexpr int BKA = 64;                       // K per A stage
    static constexpr int BKB = BN == 128 ? 32 : 64;      // K per B stage = per step
    static constexpr int NS = BN == 64 ? 4 : 2;          // buffers per operand
    static constexpr int R = BKA / BKB;                  // steps per A stage
    static constexpr int KK = BKB / 16;                  // MFMA k-steps per step
    static constexpr int WN = BN / WC;                   // columns of a wave's part
    static constexpr int NI = WN / 32;                   // 32 x 32 blocks across it
    static constexpr int kStageA = kBM * BKA * 2;        // bytes of one A buffer
    static constexpr int kStageB = BKB * BN * 2;         // bytes of one B buffer
    static constexpr int kBBase = NS * kStageA;          // B buffers follow the A buffers
    static constexpr int kLds = NS * (kStageA + kStageB);
    static constexpr int kARowBytes = BKA * 2;           // 128
    static constexpr int kAC = BKA / 8;                  // 16-byte chunks per A row
    static constexpr int kARows = 64 / kAC;              // A rows per 1-KiB load
    static constexpr int kBRowBytes = BN * 2;
    static constexpr int kBRows = 1024 / kBRowBytes;     // B rows per 1-KiB load
    static constexpr int kPart = kWM * WN;               // floats of a wave's part
    static constexpr int kTile = kBM * BN;
    static constexpr int kEpiStride = WN + 4;            // LDS floats per row of the final transpose
    static constexpr int kEpiWave = 32 * kEpiStride;     // a wave's 32-row band
    static constexpr int kWGsPerCU = BN == 128 ? 2 : 1;
    // XOR applied to the 16-byte chunk index of A row m in LDS
    static __device__ __forceinline__ int swz_a(int m) { return (m >> 1) & 7; }
    // ... and of B row k (see the LDS layout below)
    static __device__ __forceinline__ int swz_b(int k) { return BN == 64 ? 4 * ((k >> 1) & 1) : 4 * (k & 3); }
    static_assert(kLds * kWGsPerCU <= 160 * 1024, "LDS");
    static_assert(NW * kEpiWave * 4 <= kLds, "epilogue LDS");
    static_assert(NS == 2 || R == 1, "a deep pipeline stages A and B together");
};

// Fragment order of a wave's part: the part-th 4 accumulators of block (mi, ni)
// of lane l sit at byte lane * 16 + frag_soff(mi, ni, part), so one
// instruction of a wave moves 1 KiB of contiguous memory.
template <class G>
__device__ __forceinline__ unsigned frag_soff(int mi, int ni, int part) {
    return (unsigned)(((mi * G::NI + ni) * 4 + part) * 1024);
}

// LDS layout (bytes): A buffers at s kStageA (256 rows m x 64 k, 128 bytes
// per row), B buffers at kBBase + s kStageB (BKB rows k x BN n), s = 0 ..
// NS - 1; no padding.  All are filled by direct global->LDS loads (one
// instruction = 64 lanes x 16 B = 1 KiB of consecutive LDS) and spread over
// the banks by XOR-ing the 16-byte chunk index:
//   A: chunk c of row m is stored at chunk c ^ ((m >> 1) & 7)
//   B: chunk c of row k is stored at chunk c ^ (4 (k & 3)), or, for BN = 64
//      (rows of 128 bytes, two to a bank cycle), at c ^ (4 ((k >> 1) & 1))
// The LDS has 64 banks of 4 bytes and serves 16 lanes of a 16-byte read, or
// 32 lanes of an 8-byte read, per cycle; with these swizzles the 16 rows of an
// A fragment read, and the 4 rows x 2 column groups of a transposed B read,
// land on 256 distinct bytes, so neither read has a bank conflict.
__device__ __forceinline__ lds_void* lds_at(unsigned short* lds, unsigned byte) {
    return (lds_void*)((__attribute__((address_space(3))) char*)(lds_void*)lds + byte);
}

// Every buffer view a tile uses spans less than 2 GiB (a view's size is a
// 32-bit count): B (K x N bf16), a 256-row panel of A (256 x K bf16) and 128
// rows of an fp32 output tile or partial (128 x N).
inline bool gemm_views_fit(int N, int K) {
    const long long lim = 1LL << 31;
    return (long long)K * N * 2 < lim && (long long)K * kBM * 2 < lim && (long long)N * kWM * 4 < lim;
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

// Wait until at most `n` of this wave's vector memory operations are in
// flight (n rounded down to a count listed here).  The counter retires loads
// and stores together, in issue order, so this waits for every operation but
// the n issued last.
__device__ __forceinline__ void wait_vm(int n) {
    if (n >= 20) asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
    else if (n >= 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (n >= 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if (n >= 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else if (n >= 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else if (n >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (n >= 7) asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
    else if (n >= 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if (n >= 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else if (n >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (n >= 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if (n >= 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if (n >= 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Work a caller slips into the K loop of a tile (two-buffer pipeline only).
// At step t, right after the step's stage loads, issue(t) issues exactly
// ops(t) vector memory operations (both wave-uniform); the next step's wait
// lets those stay in flight, since they come after the loads it waits for.
// begin() and end(steps) bracket the loop.
struct NoHook {
    static constexpr bool kActive = false;
    __device__ __forceinline__ void begin() {}
    __device__ __forceinline__ int ops(int) const { return 0; }
    __device__ __forceinline__ void issue(int) {}
    __device__ __forceinline__ void end(int) {}
};

// C tile (tr, tc) of A B into acc (the wave's part): rows 256 tr .. of A
// (M x K row-major), columns BN tc .. of B (K x N row-major), over the K
// range kbeg .. kbeg + kl (all of K by default).  APOL is the cache policy
// of the A loads (device scope when another workgroup of the same launch
// wrote A).
//
// MFMA operands (v_mfma_f32_32x32x16_bf16): lane l holds A[m = l % 32][k =
// 8 (l / 32) + t] and B[k = 8 (l / 32) + t][n = l % 32], t = 0..7.  A is read
// with ds_read_b128 (8 consecutive k of one row).  B comes from its natural
// k-major layout through the LDS transpose read ds_read_b64_tr_b16: within
// each group of 16 lanes, when lane j points at row kb + j / 4, columns
// cb + 4 (j % 4) .. +3, lane i receives rows kb .. kb+3 of column cb + i, so
// two such reads give a lane its 8 consecutive k of one column.
//
// Accumulator v of lane l holds column l % 32, row 8 (v / 4) + 4 (l / 32) +
// v % 4 of its 32 x 32 block.
template <class G, int APOL, class Hook>
__device__ __forceinline__ void gemm_tile_h(int K, int N, const unsigned short* __restrict__ A,
                                            const unsigned short* __restrict__ B, int tr, int tc,
                                            f32x16 (&acc)[kMI][G::NI], unsigned short* lds,
                                            int lane, int wave, int wr, int wc, Hook& hook,
                                            int kbeg = 0, int kl = -1) {
    static_assert(!Hook::kActive || G::NS == 2, "K-loop work needs the two-buffer pipeline");
    constexpr int BN = G::BN;
    // Who issues the stage loads.  With the 256-wide tile only waves 0-3 do
    // (16 each), one per SIMD: all 64 loads of a step queue up at the CU's
    // address unit, and the waves that issue them stall until it takes
    // them; this way each SIMD's other wave goes straight on to its MFMAs
    // meanwhile and keeps the matrix core busy.
    constexpr int LW = BN == 256 ? G::NW / 2 : G::NW;
    constexpr int kLA = kBM / G::kARows / LW;          // this wave's loads per A stage, if it loads
    constexpr int kLB = G::BKB / G::kBRows / LW;       // ... per B stage
    static_assert(kBM % (LW * G::kARows) == 0 && G::BKB % (LW * G::kBRows) == 0, "load split");
    if (kl < 0) kl = K;
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

    // A panel: 256 rows x kl (row stride K); B panel: kl rows x BN columns
    // (row stride N); both views end at the last element the tile reads.
    const rsrc_t Av = tile_view(A + (size_t)tr * kBM * K + kbeg, ((long long)(kBM - 1) * K + kl) * 2);
    const rsrc_t Bv = tile_view(B + (size_t)kbeg * N + (size_t)tc * BN, ((long long)(kl - 1) * N + BN) * 2);

    // Direct loads.  A instruction i of loading wave w fills rows 8 (kLA w + i)
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
        const int kr = par * G::kBRows + lane / BC;        // row (mod 4) of this lane
        const int cb = (lane % BC) ^ G::swz_b(kr);
        b_voff[par] = (unsigned)(((lane / BC) * N + cb * 8) * 2);
    }
    auto issue_a = [&](int st, int slot) {                 // A stage st (K 64 st ..)
        const unsigned base = (unsigned)(slot * G::kStageA);
        if (wave >= LW) return;
#pragma unroll
        for (int i = 0; i < kLA; ++i) {
            const int r0 = (wave * kLA + i) * G::kARows;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(Av, lds_at(lds, base + r0 * G::kARowBytes), 16,
                                                     a_voff[i & 1],
                                                     (unsigned)((r0 * K + st * G::BKA) * 2), 0, APOL);
        }
    };
    auto issue_b = [&](int st, int slot) {                 // B stage st (K BKB st ..)
        const unsigned base = (unsigned)(G::kBBase + slot * G::kStageB);
        if (wave >= LW) return;
#pragma unroll
        for (int i = 0; i < kLB; ++i) {
            const int k0 = (wave * kLB + i) * G::kBRows;
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
            const int chunk = (n >> 3) ^ G::swz_b(krow);
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

    // One step of BKB of K from the A buffer at abase (its k-steps ka0 ..)
    // and the B buffer at bbase.  The reads of k-step kk + 1 are issued
    // among the MFMAs of k-step kk (one after each), each MFMA waiting only
    // for the reads it consumes.  The scheduling fences and groups hold that
    // order; left alone, the compiler pairs each read with its use through
    // one register set and exposes the LDS latency once per block.
    auto step = [&](unsigned abase, int ka0, unsigned bbase, const bf16x8 (&af0)[kMI], const bf16x8 (&bf0)[G::NI]) {
        bf16x8 af[2][kMI], bf[2][G::NI];
#pragma unroll
        for (int mi = 0; mi < kMI; ++mi) af[0][mi] = af0[mi];
#pragma unroll
        for (int ni = 0; ni < G::NI; ++ni) bf[0][ni] = bf0[ni];
#pragma unroll
        for (int kk = 0; kk < G::KK; ++kk) {
            if (kk + 1 < G::KK)
                read_frags(abase, ka0 + kk + 1, bbase, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
#pragma unroll
            for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
                for (int ni = 0; ni < G::NI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        af[kk & 1][mi], bf[kk & 1][ni], acc[mi][ni], 0, 0, 0);
            if (kk + 1 < G::KK) {
#pragma unroll
                for (int g = 0; g < kMI * G::NI; ++g) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // an MFMA,
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // then an LDS read
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int KT = kl / G::BKB;                // steps
    // The previous tile's epilogue may still be reading LDS: an LDS barrier.
    // Not __syncthreads(), whose wait for every outstanding memory operation
    // would first drain the previous tile's output stores; each path's first
    // wait below counts its own loads, which return in issue order, so the
    // stores drain while the first stage loads.
    lds_barrier();
    if constexpr (G::NS == 2) {
        // Two buffers, in steps of BKB of K: A stage p serves steps R p .. R p
        // + R - 1.  At the start of step t (after the barrier, so every wave
        // is done with step t - 1) the workgroup issues B stage t + 1 into the
        // buffer step t - 1 used and, on the first step of an A stage, A stage
        // p + 1 into the buffer A stage p - 1 used.  B goes first, so at the
        // top of the next step this wave can wait for its B loads and leave
        // the A loads of the stage after in flight (R = 2, odd steps).  Past
        // the end of K the issues re-read the last stage into the free buffer
        // (never read again).
        // The hook's operations of step t go after the loads of stage t +
        // 1, so the wait at step t + 1 leaves exactly those in flight.
        const int KA = kl / G::BKA;            // A stages
        hook.begin();
        issue_b(0, 0);
        issue_a(0, 0);
        for (int p = 0; p < KA; ++p) {
#pragma unroll
            for (int r = 0; r < G::R; ++r) {
                const int t = p * G::R + r;
                // what step t - 1 issued after B stage t: its hook work (and,
                // on the second step of an A stage, A stage p + 1 before it)
                const int later = Hook::kActive && t > 0 ? hook.ops(t - 1) : 0;
                if (r == 0) wait_vm(later);        // B stage t and A stage p have landed
                else wait_vm((wave < LW ? kLA : 0) + later);  // B stage t has; A stage p + 1 may be in flight
                lds_barrier();                     // everyone's has; buffers of step t - 1 are free
                // The first k-step's fragments are read before the loads
                // are issued, so their latency hides behind the issue.  The
                // hook's work goes after the loads.
                const unsigned abuf = (unsigned)((p & 1) * G::kStageA);
                const unsigned bbuf = (unsigned)(G::kBBase + (t & 1) * G::kStageB);
                bf16x8 af0[kMI], bf0[G::NI];
                read_frags(abuf, r * G::KK, bbuf, 0, af0, bf0);
                __builtin_amdgcn_sched_barrier(0);
                issue_b(t + 1 < KT ? t + 1 : KT - 1, (t + 1) & 1);
                if (r == 0) issue_a(p + 1 < KA ? p + 1 : KA - 1, (p + 1) & 1);
                if (Hook::kActive && hook.ops(t) > 0) {
                    __builtin_amdgcn_sched_barrier(0);   // not ahead of the stage loads
                    hook.issue(t);
                }
                __builtin_amdgcn_sched_barrier(0);
                step(abuf, r * G::KK, bbuf, af0, bf0);
            }
        }
        hook.end(KT);
    } else {
        // NS buffers, A and B staged together (R = 1): stages 0 .. NS - 2 are
        // issued up front; at the start of step t (after the barrier, so every
        // wave is done with step t - 1) stage t + NS - 1 goes into the buffer
        // step t - 1 used.  Stages past the end of K are not issued, so the
        // wait allows only the stages after t that were.  Loads return in
        // issue order and nothing else is counted (the previous tile's stores
        // are drained first), so waiting for at most (stages after t) x
        // (loads per stage) to be in flight waits for exactly stage t.
        static_assert(LW == G::NW, "every wave loads in the deep pipeline");
        constexpr int L = kLA + kLB;                // this wave's loads per stage
        wait_vm(0);
#pragma unroll
        for (int s = 0; s < G::NS - 1; ++s)
            if (s < KT) {
                issue_b(s, s);
                issue_a(s, s);
            }
        int slot = 0;                          // buffer of step t
        for (int t = 0; t < KT; ++t) {
            const int after = KT - 1 - t < G::NS - 2 ? KT - 1 - t : G::NS - 2;
            wait_vm(after * L);                // stage t has landed
            lds_barrier();                     // everyone's has; the buffer of step t - 1 is free
            const int nx = t + G::NS - 1;
            if (nx < KT) {
                const int ns = slot == 0 ? G::NS - 1 : slot - 1;
                issue_b(nx, ns);
                issue_a(nx, ns);
            }
            bf16x8 af0[kMI], bf0[G::NI];
            read_frags((unsigned)(slot * G::kStageA), 0, (unsigned)(G::kBBase + slot * G::kStageB), 0, af0, bf0);
            step((unsigned)(slot * G::kStageA), 0, (unsigned)(G::kBBase + slot * G::kStageB), af0, bf0);
            slot = slot + 1 == G::NS ? 0 : slot + 1;
        }
    }
    wait_vm(0);        // the trailing loads have landed
    __syncthreads();   // all waves are done with the stages before the epilogue uses LDS
}

// gemm_tile_h with the usual (untransposed) blocks.  Callers outside this
// header go through this wrapper: calling gemm_tile_h directly from their
// kernels' bodies, the host compilation pass rejects the template for some
// tile shapes (a substitution failure it gives no reason for).
template <class G, int APOL, class Hook>
__device__ __forceinline__ void gemm_tile_with(int K, int N, const unsigned short* __restrict__ A,
                                               const unsigned short* __restrict__ B, int tr, int tc,
                                               f32x16 (&acc)[kMI][G::NI], unsigned short* lds, int lane, int wave,
                                               int wr, int wc, Hook& hook) {
    gemm_tile_h<G, APOL>(K, N, A, B, tr, tc, acc, lds, lane, wave, wr, wc, hook);
}

template <class G, int APOL = POL_PLAIN>
__device__ __forceinline__ void gemm_tile(int K, int N, const unsigned short* __restrict__ A,
                                          const unsigned short* __restrict__ B, int tr, int tc,
                                          f32x16 (&acc)[kMI][G::NI], unsigned short* lds,
                                          int lane, int wave, int wr, int wc, int kbeg = 0, int kl = -1) {
    NoHook none;
    gemm_tile_h<G, APOL>(K, N, A, B, tr, tc, acc, lds, lane, wave, wr, wc, none, kbeg, kl);
}


// GELU in its tanh form, 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))),
// the default of jax.nn.gelu, which the tensor-parallel MLP of "TPU 与分布式
// 通信原语" (collective matmul) applies.  Since 0.5 (1 + tanh(z)) =
// 1 / (1 + 2^-s) with s = 2 z log2(e), it is x / (1 + u) for x >= 0 and
// x u / (1 + u) for x < 0, u = 2^-|s| <= 1: no cancellation in the negative
// tail.  h = s / 2 = x (c1 + c3 x^2) takes one fused multiply-add, and u is
// the square of 2^-|h| so that it stays exact down to fp32's subnormals (the
// hardware exp2 flushes results below 2^-126).  Error: about 4 roundings in
// h (an absolute 4 2^-24 |s| ln 2 in the exponent, relative in u), 1 ulp
// each for exp2 and the reciprocal, and a few roundings more.
__device__ __forceinline__ float gelu_tanh(float x) {
    // c1 = sqrt(2/pi) log2(e), c3 = 0.044715 c1
    const float h = x * __builtin_fmaf(x * x, 0.05147162f, 1.1511041f);
    const float v = __builtin_amdgcn_exp2f(-fabsf(h));
    const float u = v * v;
    const float d = __builtin_amdgcn_rcpf(1.0f + u);
    return x * (h >= 0.0f ? d : u * d);
}

// Two fp32 values -> two bf16 (round to nearest even) packed low, high
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    const f32x2v f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2v));
}

// Output element of the row-major store: the fp32 sum itself, its bf16
// rounding, or bf16(gelu(bf16(x))) -- the MLP's first layer rounds the
// product to bf16 before the activation and the activation to bf16 after.
enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_GELU_BF16 = 2 };

// Four bf16 (two dwords) -> bf16(gelu) of each.
__device__ __forceinline__ u32x2 gelu_bf16x4(const u32x2 b) {
    u32x2 h;
    h[0] = pack_bf16x2(gelu_tanh(__uint_as_float(b[0] << 16)), gelu_tanh(__uint_as_float(b[0] & 0xFFFF0000u)));
    h[1] = pack_bf16x2(gelu_tanh(__uint_as_float(b[1] << 16)), gelu_tanh(__uint_as_float(b[1] & 0xFFFF0000u)));
    return h;
}

// Four fp32 values (bits) -> four bf16 in two dwords, with the epilogue EPI.
template <int EPI>
__device__ __forceinline__ u32x2 epi_bf16x4(const u32x4 o) {
    u32x2 b;
    b[0] = pack_bf16x2(__uint_as_float(o[0]), __uint_as_float(o[1]));
    b[1] = pack_bf16x2(__uint_as_float(o[2]), __uint_as_float(o[3]));
    if constexpr (EPI == EPI_GELU_BF16) b = gelu_bf16x4(b);
    return b;
}

// Store a wave's part of a finished tile row-major: element (i, j) of the
// part goes to ob[i * ld + j], fp32 for EPI_F32 and bf16 otherwise.  With
// ADD, the same part of another tile, kept in fragment order at rv, is added
// first (device-scope loads), in fp32, before any rounding.  The partial is
// read once and the result is not read again by this launch, so both stream
// past the caches (measured: the all-gather + GEMM's fp32 output 6% faster).  Each wave turns
// its part around in its own slice of LDS (free after the K loop), 32 rows
// at a time, and writes whole row segments.
template <class G, bool ADD, int EPI = EPI_F32>
__device__ __forceinline__ void store_part_rowmajor(const f32x16 (&acc)[kMI][G::NI], rsrc_t rv, void* ob,
                                                    int ld, unsigned short* lds, int lane, int wave) {
    constexpr int OSZ = EPI == EPI_F32 ? 4 : 2;   // bytes per output element
    // per-lane offsets laundered through empty asm so they are recomputed
    // here rather than kept alive across the K loop
    unsigned lane16 = (unsigned)lane * 16u;
    asm volatile("" : "+v"(lane16));
    int lds_lane = wave * G::kEpiWave + 4 * (lane >> 5) * G::kEpiStride + (lane & 31);
    asm volatile("" : "+v"(lds_lane));
    float* stage_lane = reinterpret_cast<float*>(lds) + lds_lane;   // scatter base
    constexpr int VPR = G::WN / 4;                                  // 16-byte vectors per row
    constexpr int RPS = 64 / VPR;                                   // rows per gather step
    int lds_row = wave * G::kEpiWave + (lane / VPR) * G::kEpiStride + (lane % VPR) * 4;
    asm volatile("" : "+v"(lds_row));
    const float* gather_lane = reinterpret_cast<const float*>(lds) + lds_row;
    const rsrc_t ov = tile_view(ob, ((long long)(kWM - 1) * ld + G::WN) * OSZ);
    unsigned lane_out = (unsigned)(((lane / VPR) * ld + (lane % VPR) * 4) * OSZ);
    asm volatile("" : "+v"(lane_out));
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi) {
        u32x4 x[G::NI][4];
        if constexpr (ADD) {
#pragma unroll
            for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
                for (int part = 0; part < 4; ++part)
                    x[ni][part] = ld16s<POL_DEV | POL_NT>(rv, lane16, frag_soff<G>(mi, ni, part));
        }
#pragma unroll
        for (int ni = 0; ni < G::NI; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float cv = acc[mi][ni][v];
                float o = cv;
                if constexpr (ADD) o = __uint_as_float(x[ni][v >> 2][v & 3]) + cv;
                stage_lane[(8 * (v >> 2) + (v & 3)) * G::kEpiStride + ni * 32] = o;
            }
        // 32 rows x WN columns: in step i lane l reads 16 bytes of row
        // RPS i + l / VPR at column 4 (l % VPR).  All reads go out before
        // the first conversion, so one LDS wait covers the band (read and
        // converted one at a time, the gelu epilogue waited on each: the MLP
        // layer took about 1% longer).
        u32x4 gv[32 / RPS];
#pragma unroll
        for (int i = 0; i < 32 / RPS; ++i) gv[i] = *(const u32x4*)(gather_lane + RPS * i * G::kEpiStride);
#pragma unroll
        for (int i = 0; i < 32 / RPS; ++i) {
            const u32x4 o = gv[i];
            const unsigned at = lane_out + (unsigned)(((mi * 32 + RPS * i) * ld) * OSZ);
            if constexpr (EPI == EPI_F32) {
                st16<POL_NT>(o, ov, at);
            } else {
                st8<POL_NT>(epi_bf16x4<EPI>(o), ov, at);
            }
        }
    }
}

}  // namespace ringc

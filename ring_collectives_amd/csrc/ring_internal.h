// ring_internal.h -- internal declarations shared by the HIP translation units
// of libring_collectives.so (kernel parameter blocks, workspace layout,
// launchers).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <cstddef>

#include "ring_collectives.h"

namespace ringc {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kBlock = 256;          // threads per workgroup of the ring kernels
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kFlagStride = 16;      // ints between flags: one flag per 64 bytes
constexpr size_t kStatusBytes = 256; // error word + info, at offset 0 of a workspace
constexpr int kMinTileVecs = 4;      // smallest tile: 4 vectors of 16 B per lane

// Low-latency rounds: a value travels to the right neighbour inside an 8-byte
// word together with a ready mark, so the neighbour polls the data itself
// instead of a flag it may read only after the data was stored.  Calls whose
// chunks hold at most kLlMaxChunkBytes (and whose words take at most
// kLlMaxBytes) get a region of such words in their workspace.
constexpr size_t kLlMaxChunkBytes = 256 << 10;
constexpr size_t kLlMaxBytes = 64 << 20;
constexpr int kLlVec = 4;            // words per lane per tile position
constexpr int kLlMaxRanges = 8;      // K ranges a low-latency reduce-scatter can sum as it reads

// The status block every workspace starts with (kStatusBytes; a zero fill
// initialises it).
//   code, info      the error word: RING_OK, or the first asynchronous error
//                   (RING_ETIMEOUT, RING_EWORKSPACE, RING_EPROTOCOL) and where
//                   it happened, rank | round << 8 | min(tile, 32767) << 16.
//   at 64           the fused all-gather + GEMM's finish counter.
//   data_lo_inv,    the record of data calls have left in the workspace: the
//   data_hi         byte range [~data_lo_inv, data_hi) holds every byte some
//                   call since the last zero fill may have left non-zero
//                   (bf16 partial sums, psum slots, partial GEMM tiles).  Zero
//                   fill: ~0 and 0, an empty range.  A launch whose flags or
//                   words would lie in that range stops with RING_EWORKSPACE
//                   instead of reading stale data as set flags.
struct Status {
    int code;
    int info;
    int reserved[30];
    unsigned long long data_lo_inv;
    unsigned long long data_hi;
};
static_assert(offsetof(Status, data_lo_inv) == 128 && offsetof(Status, data_hi) == 136,
              "status block layout");
static_assert(sizeof(Status) <= kStatusBytes, "status block size");
constexpr size_t kDoneOffset = 64;   // the all-gather + GEMM finish counter

// A byte range of a workspace, as offsets from its start (hi == lo: none).
struct WsSpan {
    unsigned long long lo, hi;
};

// Parameters of one launch of the persistent chunk-step kernel.
struct RingParams {
    const void* src[RING_MAX_RANKS];  // per-rank inputs (AG: compact pieces or null)
    void* dst[RING_MAX_RANKS];        // per-rank outputs
    float* carry;                     // bf16 only: P * n fp32 partial sums
    int* flags;                       // [2(P-1)][P][T] flags, kFlagStride apart
    Status* status;                   // error word
    long long n;                      // elements per rank
    long long C;                      // elements per chunk (n / P)
    long long spin_limit;             // watchdog, in wall-clock ticks
    int P;                            // ranks
    int T;                            // tiles per chunk
    int tile;                         // elements per tile
    int k_begin, k_end;               // global rounds [k_begin, k_end)
    int waves_per_rank;               // waves working for one rank
    int vec_ok;                       // 1: every chunk/tile start is 16-byte aligned
    int compact_src;                  // all-gather from compact pieces
    int map_mode;                     // wave -> (rank, lane) mapping
    int drop_round;                   // test hook: rank 0 skips this signal (0 = off)
    // circulating psum only
    void* slots;                      // P x 2 receive slots of n elements
    int psum;                         // 1: the circulating-input psum kernel
    // bidirectional reduce-scatter only
    int bidir;                        // 1: top halves travel left, bottom halves right
    int T_top;                        // positions 0 .. T_top-1 are top-half tiles
    long long h;                      // elements in the top half of a chunk
    // fp32 reduce-scatter with a bf16 result only (kDtF32Bf16Out)
    void* out16[RING_MAX_RANKS];      // the owner's chunk, rounded once to bf16
    // low-latency rounds only: [2(P-1)][P][C] words (value | 1 << 32), or null
    unsigned long long* ll;
    // fp32 reduce-scatter with a bf16 result in the low-latency rounds only:
    // rank q's input is the sum, in order s = 0 .. nranges-1, of
    // ranges[(s P + q) n ..] (0: the input is src)
    const float* ranges;
    int nranges;
    // what this launch needs zero in the workspace at its start (its flags or
    // words) and where it leaves data (see Status)
    WsSpan ws_zero, ws_data;
    int check_flags;                  // debug: every flag must be 0 when it is set
};

// Internal element type of the ring launchers: an fp32 reduce-scatter whose
// owner stores its chunk's sum rounded once to bf16.
constexpr int kDtF32Bf16Out = 16;

// Workspace layout of the ring collectives for (P, n, dtype).
struct RingWs {
    size_t flags_off, flags_bytes;
    size_t ll_off, ll_bytes;          // low-latency words (0 bytes: calls too large for them)
    size_t carry_off, carry_bytes;    // last, so a call that needs no carry may omit it
    size_t total;
};

int elem_bytes(int dtype);
int elems_per_vec(int dtype);
// tile_elems: the tile the flag table is sized for (0: the smallest tile any
// tuning uses, so one workspace serves every tuning).
RingWs ring_ws_layout(int P, size_t n, int dtype, bool with_ll = true, size_t tile_elems = 0);

// Tuning knobs: defaults, overridable by RING_* environment variables at
// first use and by ring_set_tuning().
ring_tuning_t tuning();

// Launchers (return hipSuccess or the launch error).
hipError_t launch_copy(const void* const* src, void* const* dst, int P, size_t bytes,
                       int shift, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_ring(RingParams& prm, int dtype, int tile_vecs, int grid_blocks,
                       hipStream_t s);   // prm.bidir selects the bidirectional kernel, prm.ll the low-latency one
int ring_blocks_per_cu(int dtype, int tile_vecs, int kind);   // occupancy: 0 ring, 1 bidir, 2 psum, 3 low-latency

// The fp32 ring reduce-scatter of src into dst (the ring's partial sums; dst
// may be src), with the owner's chunk of the sum rounded once to bf16 into
// out16[q] (n / P elements) instead of stored in dst.  P >= 2.  The MLP
// layer's unfused path.
// extra: a further span of ws that the caller's other launches leave data
// in, added to the workspace's record by this launch.
int ring_reduce_scatter_bf16_out(const void* const* src, void* const* dst, void* const* out16, int P, size_t n,
                                 void* ws, size_t ws_bytes, void* stream, WsSpan extra);
// The same reduce-scatter of inputs that are each the in-order sum of S
// ranges (rank q's: ranges[(s P + q) n ..], s < S <= kLlMaxRanges), summed
// as the rounds read them.  Only in the low-latency rounds: RING_EUNSUPPORTED,
// with nothing launched, when the call does not take them.
int ring_reduce_scatter_ranges_bf16_out(const float* ranges, int S, void* const* out16, int P, size_t n,
                                        void* ws, size_t ws_bytes, void* stream, WsSpan extra);
// ring_all_gather with a further data span recorded (as above).
int ring_all_gather_rec(const void* const* src_or_null, void* const* dst, int P, size_t n, int dtype,
                        void* ws, size_t ws_bytes, void* stream, WsSpan extra);

// GEMM + reduce-scatter workspace size (n = M * N per rank).
size_t gemm_rs_workspace_bytes(int P, size_t n);
size_t ag_gemm_workspace_bytes(int P, size_t n);

// The fused GEMM launches behind the C ABI.  gemm_rs_run: epi is what out
// holds (0 the fp32 sums, 1 their bf16 rounding, 2 bf16(gelu(bf16(sum)))),
// its flags and partial tiles sit region_off bytes further into ws than in a
// call of its own (the status word stays at ws); batched makes it P
// independent products with no reduce-scatter (out[q] = A_q B_q, M % 256),
// and ksplit > 1 then splits K into that many ranges whose fp32 products go
// to split[(s P + q) M N ..] instead (epi must be EPI_F32; out unused).  ag_gemm_run: gelu_bf16 stores
// bf16(gelu(bf16(product))) instead of the fp32 product.
// Both record `extra` (a span of ws other launches of the caller leave data
// in) in the workspace's record, as well as their own data.
int gemm_rs_run(const void* const* A, const void* const* B, void* const* out, int P, int M, int N, int K,
                void* ws, size_t ws_bytes, void* stream, int epi, size_t region_off, int batched = 0,
                int ksplit = 1, float* split = nullptr, WsSpan extra = WsSpan{0, 0});
int ag_gemm_run(const void* const* A_shard, const void* const* B, void* const* A_full, void* const* C,
                int P, int M, int N, int K, void* ws, size_t ws_bytes, void* stream, int gelu_bf16,
                WsSpan extra = WsSpan{0, 0});

// Device properties cached per device.
struct DevInfo {
    int cus;
    long long wall_khz;
};
DevInfo dev_info();

}  // namespace ringc

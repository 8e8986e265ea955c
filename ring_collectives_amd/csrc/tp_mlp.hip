// tp_mlp.hip -- one tensor-parallel MLP layer from the two fused collective
// GEMMs.
//
// "TPU 与分布式通信原语" (collective matmul) writes the tensor-parallel
// X = gelu(X W1) W2 with W1 split by columns and W2 by rows; a device's view
// of one layer in a stack is
//     out_shard = ReduceScatter(gelu(AllGather(prev_shard) @ W1_i) @ W2_i),
// with the product rounded to bf16 before gelu and gelu's result rounded to
// bf16 before the second product.  Here the activation shards are row blocks
// (tokens) of X, the layout of all_gather_gemm and gemm_reduce_scatter:
//   launch 1  all_gather_gemm with the gelu epilogue:
//               x_full[r] = the ring all-gather of x_shard,
//               h[r]      = bf16(gelu(bf16(x_full[r] @ W1[r])));
//   launch 2  gemm_reduce_scatter with a bf16 epilogue:
//               out_shard[r] = bf16(rows [r M/P, (r+1) M/P) of sum_q h[q] @ W2[q]),
//               summed in fp32 in the ring's order, rounded once.
// The second launch needs every row of h[q] that one of its output tiles
// reads, i.e. whole rows of all of h's tiles, so the stream order between the
// two launches is the dependency; inside each launch the collective overlaps
// its GEMM tile by tile.
//
// Workspace: [status | all-gather panel flags | reduce-scatter flags and
// partial tiles].  Both kernels leave their flag tables zeroed, and the
// regions are disjoint, so one workspace serves any number of layers.
//
// Token counts below 256 per rank (the chapter's own 256 tokens over P = 4
// ranks make 64-row shards, less than one 256-row tile) run the same steps
// unfused, each on its own kernel, in stream order:
//   ring_all_gather of the row blocks                 -> x_full
//   every rank's product x_full @ W1 (the fused kernel's batched mode, no
//   reduce-scatter) with the gelu epilogue              -> h
//   every rank's product h @ W2 in fp32, its K split into S ranges so the
//   few tiles still fill the GPU                        -> range products
//   the fp32 ring reduce-scatter of their sums, the owner's block rounded
//   once to bf16 as the ring's last round stores it      -> out_shard
// Where the reduce-scatter runs its low-latency rounds (small chunks, as at
// the chapter's shape) it sums each input's ranges, in order, as it reads
// them: four launches.  Otherwise a kernel first sums the ranges into the
// partials and the reduce-scatter works on those in place: five.
// The arithmetic is the fused path's except for the order of the second
// product's sums over K (the ranges).
// Workspace: [status | ring flags | GEMM flags | P ring partial sums of
// M x D fp32 | S P range products of M x D fp32].
#include "gemm_core.h"
#include "ring_internal.h"

#include <hip/hip_runtime.h>

namespace ringc {
namespace {

size_t align256_mlp(size_t x) { return (x + 255) / 256 * 256; }

bool mlp_overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Does any of P buffers of `na` bytes at a[] overlap any of b[]?
bool any_overlap(const void* const* a, size_t na, const void* const* b, size_t nb, int P) {
    for (int i = 0; i < P; ++i)
        for (int j = 0; j < P; ++j)
            if (mlp_overlap(a[i], na, b[j], nb)) return true;
    return false;
}

bool fused_shape(int P, int M) { return M % (256 * P) == 0; }

constexpr int kMaxSplit = 8;
static_assert(kMaxSplit <= kLlMaxRanges, "the low-latency reduce-scatter sums every range");

// K ranges of the unfused second product: about 256 work items of 256 x 64
// tiles in all (one per CU; the product's automatic tile width then takes
// 64-wide tiles, as it does below one 128-wide item per CU), at most
// kMaxSplit, each range a multiple of 64.  Every range's fp32 product is
// written and read back once, so more ranges than the CUs need cost traffic.
int mlp_split(int P, int M, int D, int F) {
    const int Fr = F / P;
    const long long tiles = (long long)P * (M / 256) * (D / 64);
    int S = 1;
    while (S < kMaxSplit && tiles * S * 2 <= 256 && Fr % (64 * S * 2) == 0) S *= 2;
    return S;
}

struct MlpWs {
    // fused: where the reduce-scatter's flags start.  unfused: where the
    // GEMMs' flags, the partials and the range products start.  Bytes in all.
    size_t rs_off, gemm_off, part_off, split_off, total;
};

bool mlp_ws_layout(int P, int M, int D, int F, MlpWs& w) {
    const int Fr = F / P;
    if (fused_shape(P, M)) {
        const size_t ag = ag_gemm_workspace_bytes(P, (size_t)M * Fr);
        const size_t rs = gemm_rs_workspace_bytes(P, (size_t)M * D);
        if (!ag || !rs) return false;
        w.rs_off = align256_mlp(ag);
        w.gemm_off = w.part_off = w.split_off = 0;
        w.total = w.rs_off + rs - kStatusBytes;   // the status block is shared
        return true;
    }
    const size_t nd = (size_t)M * D;
    const size_t ring = ring_workspace_bytes(RING_OP_REDUCE_SCATTER, P, nd, RING_F32);
    const size_t ring_ag = ring_workspace_bytes(RING_OP_ALL_GATHER, P, nd, RING_BF16);
    const size_t g1 = gemm_rs_workspace_bytes(1, (size_t)M * Fr), g2 = gemm_rs_workspace_bytes(1, nd);
    if (!ring || !ring_ag || !g1 || !g2) return false;
    w.rs_off = 0;
    w.gemm_off = align256_mlp(ring > ring_ag ? ring : ring_ag);
    w.part_off = align256_mlp(w.gemm_off + (g1 > g2 ? g1 : g2) - kStatusBytes);
    w.split_off = w.part_off + (size_t)P * nd * sizeof(float);
    w.total = w.split_off + (size_t)mlp_split(P, M, D, F) * P * nd * sizeof(float);
    return true;
}

bool mlp_shape_ok(int P, int M, int D, int F) {
    return M % P == 0 && M % 256 == 0 && D % 128 == 0 && F % (128 * P) == 0;
}

// part[q][i] = sum over s = 0 .. S-1, in that order, of split[s P + q][i]
// (n a multiple of 4; 16-byte accesses, all S loads of a vector in flight).
struct PartTab {
    float* p[RING_MAX_RANKS];
};

__global__ __launch_bounds__(256) void sum_ranges_kernel(const float* split, PartTab t, int P, int S,
                                                             long long n) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int q = blockIdx.y;
    f4* out = (f4*)t.p[q];
    const long long nv = n / 4;
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nv;
         i += (long long)gridDim.x * blockDim.x) {
        f4 x[kMaxSplit];
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s)
            if (s < S) x[s] = __builtin_nontemporal_load((const f4*)(split + ((size_t)s * P + q) * n) + i);
        f4 a = x[0];
#pragma unroll
        for (int s = 1; s < kMaxSplit; ++s)
            if (s < S) a = a + x[s];
        out[i] = a;
    }
}

int mlp_unfused(const void* const* x_shard, const void* const* W1, const void* const* W2,
                void* const* x_full, void* const* h, void* const* out_shard, int P, int M, int D, int F,
                void* ws, size_t ws_bytes, const MlpWs& lay, void* stream) {
    const int Fr = F / P;
    const size_t nd = (size_t)M * D;
    // the partial sums and range products stay in the workspace: every
    // launch adds that span to the workspace's record
    const WsSpan data{lay.part_off, lay.total};
    int rc = ring_all_gather_rec(x_shard, x_full, P, nd, RING_BF16, ws, lay.gemm_off, stream, data);
    if (rc != RING_OK) return rc;
    void* part[RING_MAX_RANKS];
    for (int q = 0; q < P; ++q) part[q] = (char*)ws + lay.part_off + (size_t)q * nd * sizeof(float);
    const size_t goff = lay.gemm_off - kStatusBytes;   // the GEMMs' flags after the ring's
    // every rank's product in one launch each (the batched mode of the fused kernel)
    rc = gemm_rs_run((const void* const*)x_full, W1, h, P, M, Fr, D, ws, lay.part_off, stream, EPI_GELU_BF16,
                     goff, 1, 1, nullptr, data);
    if (rc != RING_OK) return rc;
    const int S = mlp_split(P, M, D, F);
    float* split = (float*)((char*)ws + lay.split_off);
    rc = gemm_rs_run((const void* const*)h, W2, part, P, M, D, Fr, ws, lay.part_off, stream, EPI_F32, goff, 1,
                     S, S > 1 ? split : nullptr, data);
    if (rc != RING_OK) return rc;
    if (S > 1) {
        // Where the reduce-scatter takes its low-latency rounds it sums the
        // ranges itself as it reads them, in the same order; otherwise a
        // kernel sums them into the partials first.
        rc = ring_reduce_scatter_ranges_bf16_out(split, S, out_shard, P, nd, ws, lay.gemm_off, stream, data);
        if (rc != RING_EUNSUPPORTED) return rc;
        PartTab pt;
        for (int q = 0; q < P; ++q) pt.p[q] = (float*)part[q];
        long long blocks = ((long long)nd + 255) / 256;
        if (blocks > 1024) blocks = 1024;
        hipLaunchKernelGGL(sum_ranges_kernel, dim3((unsigned)blocks, (unsigned)P), dim3(256), 0,
                           (hipStream_t)stream, split, pt, P, S, (long long)nd);
        if (hipGetLastError() != hipSuccess) return RING_EHIP;
    }
    // in place: a rank's chunk is rewritten only in a round after the ones
    // that read it as input
    return ring_reduce_scatter_bf16_out((const void* const*)part, part, out_shard, P, nd, ws, lay.gemm_off,
                                        stream, data);
}

}  // namespace
}  // namespace ringc

using namespace ringc;

extern "C" size_t tp_mlp_workspace_bytes(int P, int M, int D, int F) {
    if (P < 1 || P > RING_MAX_RANKS || M <= 0 || D <= 0 || F <= 0) return 0;
    if (!mlp_shape_ok(P, M, D, F)) return 0;
    MlpWs w;
    return mlp_ws_layout(P, M, D, F, w) ? w.total : 0;
}

extern "C" int tp_mlp_layer(const void* const* x_shard, const void* const* W1, const void* const* W2,
                            void* const* x_full, void* const* h, void* const* out_shard, int P, int M,
                            int D, int F, void* ws, size_t ws_bytes, void* stream) {
    if (P < 1 || P > RING_MAX_RANKS || M < 0 || D < 0 || F < 0) return RING_EINVAL;
    if (!x_shard || !W1 || !W2 || !x_full || !h || !out_shard) return RING_EINVAL;
    if (M == 0 || D == 0 || F == 0) return RING_OK;
    if (!mlp_shape_ok(P, M, D, F)) return RING_EUNSUPPORTED;
    for (int r = 0; r < P; ++r)
        if (!x_shard[r] || !W1[r] || !W2[r] || !x_full[r] || !h[r] || !out_shard[r]) return RING_EINVAL;
    const int Fr = F / P;
    const size_t shard_b = (size_t)(M / P) * D * 2, full_b = (size_t)M * D * 2;
    const size_t w1_b = (size_t)D * Fr * 2, w2_b = (size_t)Fr * D * 2, h_b = (size_t)M * Fr * 2;
    // h is written while x_full, x_shard and W1 are read; out_shard while h
    // and W2 are read (it may share memory with x_shard, which is no longer
    // read by then, so layers can run in place)
    if (any_overlap(h, h_b, x_full, full_b, P) || any_overlap(h, h_b, x_shard, shard_b, P) ||
        any_overlap(h, h_b, W1, w1_b, P) || any_overlap(h, h_b, W2, w2_b, P))
        return RING_EINVAL;
    for (int a = 0; a < P; ++a)
        for (int b = a + 1; b < P; ++b)
            if (mlp_overlap(h[a], h_b, h[b], h_b) || mlp_overlap(out_shard[a], shard_b, out_shard[b], shard_b))
                return RING_EINVAL;
    if (any_overlap(out_shard, shard_b, h, h_b, P) || any_overlap(out_shard, shard_b, W2, w2_b, P))
        return RING_EINVAL;
    MlpWs lay;
    if (!mlp_ws_layout(P, M, D, F, lay)) return RING_EUNSUPPORTED;
    if (!ws || ((uintptr_t)ws & 255) || ws_bytes < lay.total) return RING_EWORKSPACE;
    for (int r = 0; r < P; ++r)
        if (mlp_overlap(ws, ws_bytes, h[r], h_b) || mlp_overlap(ws, ws_bytes, x_full[r], full_b) ||
            mlp_overlap(ws, ws_bytes, out_shard[r], shard_b))
            return RING_EINVAL;

    if (!fused_shape(P, M))
        return mlp_unfused(x_shard, W1, W2, x_full, h, out_shard, P, M, D, F, ws, ws_bytes, lay, stream);
    int rc = ag_gemm_run(x_shard, W1, x_full, h, P, M, Fr, D, ws, lay.rs_off, stream, 1);
    if (rc != RING_OK) return rc;
    // gemm_rs_run's own layout puts its flags kStatusBytes in; shift them to rs_off
    return gemm_rs_run((const void* const*)h, W2, out_shard, P, M, D, Fr, ws, ws_bytes, stream, EPI_BF16,
                       lay.rs_off - kStatusBytes);
}

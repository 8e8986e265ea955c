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
// Workspace: [status | all-gather slice flags | reduce-scatter flags and
// partial tiles].  Both kernels leave their flag tables zeroed, and the
// regions are disjoint, so one workspace serves any number of layers.
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

struct MlpWs {
    size_t rs_off, total;   // where the reduce-scatter's flags start; bytes in all
};

bool mlp_ws_layout(int P, int M, int D, int F, MlpWs& w) {
    const int Fr = F / P;
    const size_t ag = ag_gemm_workspace_bytes(P, (size_t)M * Fr);
    const size_t rs = gemm_rs_workspace_bytes(P, (size_t)M * D);
    if (!ag || !rs) return false;
    w.rs_off = align256_mlp(ag);
    w.total = w.rs_off + rs - kStatusBytes;   // the status block is shared
    return true;
}

bool mlp_shape_ok(int P, int M, int D, int F) {
    return M % (256 * P) == 0 && D % 128 == 0 && F % (128 * P) == 0;
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

    int rc = ag_gemm_run(x_shard, W1, x_full, h, P, M, Fr, D, ws, lay.rs_off, stream, 1);
    if (rc != RING_OK) return rc;
    // gemm_rs_run's own layout puts its flags kStatusBytes in; shift them to rs_off
    return gemm_rs_run((const void* const*)h, W2, out_shard, P, M, D, Fr, ws, ws_bytes, stream, 1,
                       lay.rs_off - kStatusBytes);
}

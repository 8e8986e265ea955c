/*
 * ring_collectives.h -- C ABI of libring_collectives.so: ring collectives over
 * P virtual ranks whose buffers all live in the HBM of one MI355X (gfx950).
 *
 * Virtual rank r's buffer is bufs[r]; a kernel working for rank r touches
 * only its own buffers and those of its left neighbour (r - 1 + P) mod P, and
 * it synchronises with that neighbour through per-tile flags in device memory
 * (no barrier across ranks).  This is the symmetric-buffer picture of the
 * "Triton-distributed 语义" page ("对称内存模型": the same buffer exists on
 * every rank and a rank may address a peer's copy), with "the peer's copy"
 * being another slice of the same HBM.
 *
 * Conventions shared by every entry point
 *   - P        number of ranks, 1 <= P <= RING_MAX_RANKS.
 *   - n        elements per rank.  The ring splits a rank buffer into P equal
 *              chunks of C = n / P elements, so P must divide n ("全归约 3：
 *              Ring——每步大小恒定", section "Run it").  Chunk c is the flat,
 *              contiguous run [c*C, (c+1)*C).  n == 0 is a no-op.
 *   - src/dst  host arrays of P device pointers (read during the call only).
 *              Device pointers must be 4-byte aligned (2 for bf16); 16-byte
 *              alignment of every chunk start enables the 128-bit path.
 *   - dtype    RING_F32, RING_BF16 or RING_I32.  fp32 additions are IEEE
 *              round-to-nearest-even in the ring's fixed order; int32 adds
 *              wrap modulo 2^32; bf16 is added in fp32 (see below).
 *   - ws       device workspace of at least ring_workspace_bytes(...) bytes,
 *              256-byte aligned, owned by the caller.  It must be
 *              zero-filled once before its first use (ring_workspace_init,
 *              or any zero fill); every call that completes normally leaves
 *              its flags and low-latency words zero again, so back-to-back
 *              calls on one stream need no re-initialisation.  Some calls
 *              also leave data in the workspace: the fp32 partial sums of a
 *              bf16 reduce-scatter or all-reduce in the flag rounds, the
 *              receive slots of the circulating psum, the partial tiles of
 *              the fused GEMMs and the MLP layer.  The workspace's first 256
 *              bytes keep a record of where such data lies; a later call
 *              whose flags or words would lie there (another shape or
 *              operation on the same workspace) stops at once and reports
 *              RING_EWORKSPACE through ring_last_error, with its outputs
 *              undefined, instead of reading that data as flags.  A zero
 *              fill clears the record.  Calls of one shape and operation
 *              never trip it.  Calls that share a workspace must be ordered
 *              (same stream).
 *   - stream   a hipStream_t passed as void* (NULL = the default stream).
 *              Every call is asynchronous on that stream; nothing is
 *              allocated, printed or thrown by the library.  A call
 *              records no memset and leaves its flags zeroed, so it can be
 *              captured in a HIP graph and the graph replayed like the
 *              call.
 *
 * Errors: argument errors are returned synchronously (RING_EINVAL,
 * RING_EUNSUPPORTED, RING_EWORKSPACE); a failed HIP launch returns RING_EHIP.
 * A rank that waits for its neighbour longer than the watchdog limit
 * (default 5 s) stops, records RING_ETIMEOUT in the workspace and makes the
 * other ranks stop too; ring_last_error() reports it.
 *
 * Residency: the ring calls' waves wait only within the ring of one tile
 * position (P consecutive waves of the launch), so they progress with part
 * of their grid resident, e.g. beside other kernels on other streams.  In
 * the two fused GEMM calls and tp_mlp_layer, workgroups wait for other
 * workgroups of the same launch, so all of them must get to run: beside a
 * kernel that holds part of the GPU a launch is delayed until that kernel's
 * workgroups finish (within the watchdog limit), and two such calls must
 * not run at once on different streams.  Asynchronous errors
 * (RING_ETIMEOUT, RING_EWORKSPACE from the record above, RING_EPROTOCOL
 * from the debug check_flags knob) leave the outputs undefined; the
 * workspace must then be re-initialised.
 */
#ifndef RING_COLLECTIVES_H
#define RING_COLLECTIVES_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RING_MAX_RANKS 64

typedef enum { RING_F32 = 0, RING_BF16 = 1, RING_I32 = 2 } ring_dtype_t;

typedef enum {
    RING_OP_PPERMUTE = 0,
    RING_OP_REDUCE_SCATTER = 1,
    RING_OP_ALL_GATHER = 2,
    RING_OP_ALL_REDUCE = 3,
    RING_OP_GEMM_REDUCE_SCATTER = 4,
    RING_OP_REDUCE_SCATTER_BIDIR = 5,
    RING_OP_ALL_GATHER_GEMM = 6,
    RING_OP_PSUM_CIRCULATING = 7
} ring_op_t;

enum {
    RING_OK = 0,
    RING_EINVAL = -1,       /* bad rank count, size, pointer or alignment   */
    RING_EUNSUPPORTED = -2, /* bad dtype or a shape this version rejects    */
    RING_EWORKSPACE = -3,   /* workspace missing or too small               */
    RING_EHIP = -4,         /* a HIP runtime call failed                    */
    RING_ETIMEOUT = -5,     /* a rank waited past the watchdog limit        */
    RING_EPROTOCOL = -6     /* debug check: a flag was set a second time    */
};

/*
 * Bytes of workspace a call needs.  op is a ring_op_t.  For
 * RING_OP_GEMM_REDUCE_SCATTER and RING_OP_ALL_GATHER_GEMM pass n = M * N
 * (elements of one rank's product) and dtype RING_F32.  Returns 0 for invalid arguments (and for ppermute,
 * which needs none).
 * The one-way ring collectives of small calls (chunks of at most 256 KiB,
 * and 2 (P - 1) n at most 8 Mi) also get one 8-byte word per element and
 * round of the ring, 16 (P - 1) n bytes: the low-latency rounds (see
 * ll_max_chunk_bytes below) pass every value on in such a word, together
 * with its ready mark, instead of behind a per-tile flag.  A call runs them
 * only when its workspace holds those words; a smaller workspace that holds
 * its flag table (one sized for a larger call, say) serves it with the flag
 * rounds.
 */
size_t ring_workspace_bytes(int op, int P, size_t n, int dtype);

/* Zero-fill a workspace on `stream` (a fill kernel, usable under graph
 * capture).  Returns RING_OK or RING_EINVAL / RING_EHIP. */
int ring_workspace_init(void *ws, size_t ws_bytes, void *stream);

/*
 * ppermute (right shift): every rank sends its whole buffer to its right
 * neighbour, so on return dst[r] holds what src[(r - 1 + P) mod P] held.
 * "Pallas TPU Distributed Collectives 复习文档", section 1 (right-shift
 * example, checked against lax.ppermute with perm (i, i+1 mod P)).
 * n elements per rank of `dtype` (a bit copy; dtype only sets the element
 * size); P need not divide n here.  dst and src buffers must not overlap.
 * No workspace.
 */
int ring_ppermute(const void *const *src, void *const *dst, int P, size_t n,
                  int dtype, void *stream);

/*
 * Ring reduce-scatter, P-1 rounds ("全归约 3：Ring——每步大小恒定",
 * Walkthrough, first loop; the same schedule as the reduce-scatter kernel of
 * "TPU 与分布式通信原语").  In round s = 0..P-2 rank r takes chunk
 * c = (r - s - 2) mod P from its left neighbour -- the neighbour's input at
 * s = 0, otherwise the partial sum the neighbour stored in round s-1 -- adds
 * its own input chunk c and stores the result as its chunk c.
 *
 * On return chunk r of dst[r] holds the sum over all ranks of chunk r
 * (psum_scatter's result: "Pallas TPU Distributed Collectives 复习文档",
 * section 4.4).  The other chunks of dst[r] hold partial sums (unspecified).
 * fp32 order: chunk c is ((x_{c+1} + x_{c+2}) + ...) + x_c, indices mod P.
 * bf16: partial sums travel in fp32 through the workspace; the owner rounds
 * its final fp32 sum once to bf16 (nearest, ties to even).
 * In place (dst[r] == src[r] for every r) is allowed; otherwise src and dst
 * must not overlap.
 */
int ring_reduce_scatter(const void *const *src, void *const *dst, int P, size_t n,
                        int dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * Bidirectional ring reduce-scatter, P steps ("Pallas TPU Distributed
 * Collectives 复习文档", section 4, lax.psum_scatter, and its walk-through in
 * 4.6).  Every chunk is split into a top half (its first C - C/2 elements),
 * which travels to the left neighbour, and a bottom half, which travels to
 * the right one, so both directions of every ring link carry half the data.
 * At step s = 0..P-2 rank r takes the top half of chunk (r + s + 1) mod P
 * from its right neighbour (that neighbour's input at s = 0, otherwise the
 * partial sum it stored at step s-1) and adds its own input; likewise the
 * bottom half of chunk (r - s - 1) mod P from its left neighbour.  At step
 * P-1 the halves of chunk r arrive complete and are stored unchanged.
 *
 * On return chunk r of dst[r] holds the sum over all ranks of chunk r, as for
 * ring_reduce_scatter; the other chunks of dst[r] hold partial sums
 * (unspecified).  fp32 order, owner first: top half of chunk c is
 * ((x_c + x_{c-1}) + ...) + x_{c+1}, bottom half ((x_c + x_{c+1}) + ...) +
 * x_{c-1}, indices mod P.  bf16: partial sums travel in fp32 through the
 * workspace and the complete half is rounded once to bf16.  In place is
 * allowed as for ring_reduce_scatter.  Workspace: RING_OP_REDUCE_SCATTER_BIDIR.
 */
int ring_reduce_scatter_bidir(const void *const *src, void *const *dst, int P, size_t n,
                              int dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * Circulating-input psum ("Pallas TPU Distributed Collectives 复习文档",
 * section 3, lax.psum, and its walk-through in 3.5): every rank's whole
 * input travels once around the ring to the right, and each rank adds what
 * arrives into an accumulator that starts at zero, so
 *     dst[r] = (((0 + src[r-1]) + src[r-2]) + ...) + src[r]   (indices mod P)
 * -- every rank ends with the sum over ranks, each in its own order.  Items
 * move through two receive slots per rank in the workspace, and a rank
 * writes its neighbour's slot only after the neighbour has flagged it free
 * (the page's capacity semaphore).  It moves P times a rank's buffer per
 * rank, against 2(P-1)/P for ring_all_reduce: the page's teaching contrast.
 * bf16: the inputs circulate unchanged, the accumulator is fp32, the result
 * is rounded once.  P need not divide n.  In place (dst[r] == src[r]) is
 * allowed.  Workspace: RING_OP_PSUM_CIRCULATING.
 */
int ring_psum_circulating(const void *const *src, void *const *dst, int P, size_t n,
                          int dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * Ring all-gather, P-1 rounds ("全归约 3", Walkthrough, second phase; the
 * slot rule of "Pallas TPU Distributed Collectives 复习文档", section 2).
 * In round t = 0..P-2 rank r copies chunk (r - t - 1) mod P of its left
 * neighbour into the same chunk of its own buffer.
 *
 * If src_or_null is NULL, chunk r of dst[r] must already hold rank r's piece
 * (the in-place form that follows a reduce-scatter).  Otherwise src_or_null[r]
 * points at rank r's compact piece of C = n / P elements, which is placed at
 * chunk r of dst[r] (the pieces must not overlap dst).  On return every
 * dst[r] is the concatenation of the P pieces in rank order.
 */
int ring_all_gather(const void *const *src_or_null, void *const *dst, int P, size_t n,
                    int dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * Ring all-reduce = reduce-scatter then all-gather, 2(P-1) rounds in one
 * launch ("全归约 3", The idea and Walkthrough: one signal row per round,
 * rows 0..P-2 for the first phase and P-1..2P-3 for the second).  On return
 * every dst[r] holds the sum over ranks of src[q] (every rank the same bits).
 * In place allowed as for ring_reduce_scatter.
 */
int ring_all_reduce(const void *const *src, void *const *dst, int P, size_t n,
                    int dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * GEMM + reduce-scatter with tile-level overlap ("Triton-distributed 语义",
 * "GEMM + ReduceScatter 重叠": the GEMM produces output tiles and signals each
 * one; the reduce-scatter consumes tiles as their signals arrive; and
 * "TPU 与分布式通信原语", collective matmul, for the unfused meaning).
 *
 * A[r]: bf16 M x K row-major, B[r]: bf16 K x N row-major, for every rank r.
 * out[r]: fp32 (M / P) x N row-major = rows [r M/P, (r+1) M/P) of
 * sum_q A[q] B[q].  The per-rank products are accumulated in fp32 on the
 * matrix cores; the sum over ranks follows the fp32 ring reduce-scatter over
 * row-block chunks (chunk c = rows [c M/P, (c+1) M/P)).
 * Shapes this version accepts: M % (256 P) == 0, N % 128 == 0, K % 64 == 0,
 * and K N < 2^30, K < 2^22, N < 2^22 (every view a tile uses, B and 256-row
 * panels of A and of the output, below 2 GiB); others: RING_EUNSUPPORTED.
 * Output tiles are 256 x 256, 256 x 128 or 256 x 64 (see gemm_tile_n
 * below); results are the same bits either way.  Workgroups wait for
 * other workgroups of the launch (see Residency above); a wait that
 * outlives the watchdog ends in RING_ETIMEOUT.
 */
int gemm_reduce_scatter(const void *const *A, const void *const *B, void *const *out,
                        int P, int M, int N, int K, void *ws, size_t ws_bytes,
                        void *stream);

/*
 * All-gather + GEMM with tile-level overlap ("Triton-distributed 语义",
 * "AllGather + GEMM 重叠": GEMM tiles wait for the blocks they need and start
 * as soon as they arrive, every rank starting on its local block; "TPU 与分布式
 * 通信原语", collective matmul, all-gather-matmul, for the unfused meaning).
 *
 * A_shard[r]: bf16 (M / P) x K row-major, rank r's row block of A.
 * B[r]: bf16 K x N row-major.  A_full[r]: bf16 M x K, written: on return it
 * holds the ring all-gather of the row blocks (block c at rows
 * [c M/P, (c+1) M/P)).  C[r]: fp32 M x N row-major, written: A_full @ B[r],
 * accumulated in fp32 on the matrix cores.  The blocks travel the ring of
 * ring_all_gather (rank r receives block (r - t - 1) mod P in round t); rank
 * r's GEMM handles block r first, then the blocks in the order they arrive.
 * A_full buffers must not overlap the shards or each other.  Workgroups
 * wait for other workgroups of the launch (see Residency above); a wait
 * that outlives the watchdog ends in RING_ETIMEOUT.
 * Shapes this version accepts: M % (256 P) == 0, N % 128 == 0, K % 64 == 0,
 * and K N < 2^30, K < 2^22, N < 2^22 (every view a tile uses, B and 256-row
 * panels of A and of the output, below 2 GiB); others: RING_EUNSUPPORTED.
 */
int all_gather_gemm(const void *const *A_shard, const void *const *B, void *const *A_full,
                    void *const *C, int P, int M, int N, int K, void *ws, size_t ws_bytes,
                    void *stream);

/*
 * One tensor-parallel MLP layer, out = ReduceScatter(gelu(AllGather(x) @ W1_r)
 * @ W2_r) ("TPU 与分布式通信原语", collective matmul: the tensor-parallel
 * X = gelu(X @ W1) @ W2 with W1 split by columns and W2 by rows, and the
 * multi-layer form in which each layer starts from the previous layer's
 * shard).  gelu is the tanh form, 0.5 x (1 + tanh(sqrt(2/pi)(x + 0.044715
 * x^3))); as on that page the first product is rounded to bf16 before gelu
 * and gelu's result to bf16 before the second product.
 *
 * Shapes: M tokens, model width D, hidden width F (all ranks together).
 * x_shard[r]: bf16 (M / P) x D, rows [r M/P, (r+1) M/P) of the layer input.
 * W1[r]: bf16 D x (F / P), column block r of W1.  W2[r]: bf16 (F / P) x D,
 * row block r of W2.  Written: x_full[r] (bf16 M x D, the gathered input),
 * h[r] (bf16 M x (F / P), bf16(gelu(bf16(x_full[r] @ W1[r])))), and
 * out_shard[r] (bf16 (M / P) x D): rows [r M/P, (r+1) M/P) of
 * sum_q h[q] @ W2[q], accumulated in fp32 (products on the matrix cores, the
 * sum over ranks in the ring reduce-scatter's order) and rounded once.
 * Runs as two launches on `stream`: all_gather_gemm with the gelu epilogue,
 * then gemm_reduce_scatter with a bf16 epilogue.  out_shard may be the same
 * memory as x_shard (a layer in place); h must not overlap any input, x_full
 * or another h; out_shard must not overlap h or W2; none may overlap ws.
 * ws: at least tp_mlp_workspace_bytes(P, M, D, F) bytes, 256-byte aligned,
 * zeroed once; ring_last_error reports a watchdog timeout of any launch.
 * Shapes this version accepts: M % 256 == 0, M % P == 0, D % 128 == 0,
 * F % (128 P) == 0.  With M % (256 P) != 0 (fewer than 256 tokens per rank,
 * as at the chapter's own 256 tokens over 4 ranks) the same steps run
 * unfused, in separate launches: ring_all_gather; every rank's first product
 * (gelu epilogue); every rank's second product in fp32 into the workspace,
 * its K split into up to 8 ranges so the few output tiles still fill the
 * GPU; and the fp32 ring reduce-scatter of each rank's sum of its ranges
 * (summed in order as the ring reads them where its low-latency rounds run,
 * else by a kernel first), the owner's block rounded once to bf16.  That
 * arithmetic differs from the fused path's only in the order of the second
 * product's sums over K (the ranges), within the same error bound;
 * integer-valued operands give the same bits.
 */
int tp_mlp_layer(const void *const *x_shard, const void *const *W1, const void *const *W2,
                 void *const *x_full, void *const *h, void *const *out_shard, int P, int M, int D,
                 int F, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of tp_mlp_layer; 0 for invalid or unsupported shapes. */
size_t tp_mlp_workspace_bytes(int P, int M, int D, int F);

/*
 * Synchronises `stream` and returns the error word a kernel left in `ws`
 * (RING_OK if none).  If info is not NULL it receives where the error
 * happened, rank | round << 8 | tile << 16 (tile saturates): the stuck
 * wait for RING_ETIMEOUT, the flag set twice for RING_EPROTOCOL, 0 for
 * RING_EWORKSPACE.  ws_bytes is the workspace's size (at least 256).
 */
int ring_last_error(const void *ws, size_t ws_bytes, void *stream, int *info);

/* Static description of an error code. */
const char *ring_strerror(int code);

/*
 * Tuning and debug knobs of the chunk-step kernel, process-wide.  Changing
 * them while calls are in flight is not supported.  Results never depend on
 * them (fp32 bits included); only speed does, except for the debug hooks.
 *   tile_vecs      16-byte vectors per lane per tile: 4, 8 or 16 (default;
 *                  a tile is the unit of one flag: 64 lanes x tile_vecs x 16
 *                  bytes).
 *   waves_per_cu   resident wavefronts to aim for per compute unit (4..16;
 *                  never more than half the occupancy limit is used).
 *   map_mode       wavefront -> (rank, tile) mapping: 0 the P ranks of a tile
 *                  position in consecutive wavefronts, 2 a tile position's
 *                  whole ring on one XCD.
 *   timeout_s      watchdog for one wait, seconds (> 0).
 *   stepwise       1: one launch per round, ordered by the stream instead of
 *                  flags (the "inject a barrier between steps" debugging aid
 *                  of "Triton-distributed 语义", best practice 8).
 *   drop_round     test hook: if >= 1, rank 0 never signals round drop_round
 *                  (all_gather_gemm: never flags its tiles of that phase),
 *                  so the waits on it must end in RING_ETIMEOUT.
 *   gemm_tile_n    output tile width of the fused GEMMs: 128 (two 4-wave
 *                  workgroups per compute unit), 64 (one 4-wave workgroup
 *                  with a deeper load pipeline; all_gather_gemm takes 128
 *                  for 64), 256 (one 8-wave workgroup; needs N % 256 ==
 *                  0), or 0 to choose per call: 256 when the 256 x 256
 *                  tiles give every compute unit work (for
 *                  gemm_reduce_scatter, counting the tiles of all phases;
 *                  for all_gather_gemm, those of one chunk per rank), else
 *                  64 when the 256 x 64 ones number at most one per
 *                  compute unit (gemm_reduce_scatter and tp_mlp_layer),
 *                  else 128.
 *   ll_max_chunk_bytes  the one-way reduce-scatter, all-gather and
 *                  all-reduce run their rounds in the low-latency form when
 *                  a chunk (n / P elements) takes at most this many bytes
 *                  and the workspace holds the words (see
 *                  ring_workspace_bytes); 0 turns that off.  0 .. 262144
 *                  (default).  Same chunks, same additions, same results;
 *                  a round costs about half the latency.  Not in stepwise
 *                  mode.
 *   check_flags    debug: 1 makes every flag set (ring rounds, psum,
 *                  GEMM tiles, all-gather panel shares) an atomic add that
 *                  returns the flag's old value, which must be 0 -- each
 *                  flag of a launch is set exactly once and cleared by its
 *                  reader ("全归约 3：Ring——每步大小恒定", Walkthrough: a
 *                  Ge(1) wait on a row notified once) -- and every
 *                  low-latency word be empty before it is written.  A
 *                  violation is recorded as RING_EPROTOCOL with its (rank,
 *                  round, tile).  Results are unchanged; 0 (default) off.
 */
typedef struct {
    int tile_vecs;
    int waves_per_cu;
    int map_mode;
    double timeout_s;
    int stepwise;
    int drop_round;
    int gemm_tile_n;
    int ll_max_chunk_bytes;
    int check_flags;
} ring_tuning_t;

void ring_get_tuning(ring_tuning_t *t);
int ring_set_tuning(const ring_tuning_t *t);   /* RING_EINVAL on bad values */

/*
 * ring_all_reduce for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it): the same
 * call without a workspace argument.  Its flags, low-latency words and bf16
 * partial sums live in a static device array of RING_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends;
 * the call allocates nothing and calls no allocating routine.  Results are
 * the same bits as ring_all_reduce's.
 *
 * Each call first clears the part of that array it needs zero (a fill
 * kernel on `stream`, no memset), so no call depends on what an earlier one
 * left there.  Every call on one device shares the one array: calls that
 * overlap in time on one device (different streams, or host threads) race
 * and give undefined results; order them.
 *
 * The flag table is sized for the tile the call actually uses (16 KiB tiles
 * by default), plus, for bf16, P n fp32 partial sums; a call that needs more
 * than RING_NOALLOC_SCRATCH_BYTES returns RING_EWORKSPACE synchronously and
 * launches nothing (at the default tuning: fp32 and int32 up to about 73 Mi
 * elements per rank at P = 8, bf16 up to about 0.5 Mi).  Other argument
 * errors as ring_all_reduce.  A watchdog timeout leaves the outputs
 * undefined and is not reported (there is no workspace to read it from);
 * the next call starts from a cleared array.
 */
#define RING_NOALLOC_SCRATCH_BYTES (16u << 20)
int ring_all_reduce_noalloc(const void *const *src, void *const *dst, int P, size_t n,
                            int dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RING_COLLECTIVES_H */

/*
 * ring_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded CPU oracle for the ring collectives.  It is
 * the yardstick the GPU library is checked against and shares no code, header,
 * table or constant with it.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.
 *
 * Build (done by oracle/__init__.py or __graft_entry__.build()):
 *     gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 *
 * Data model.  P ranks; every rank holds n elements; the P rank buffers sit
 * back to back in one host array ("rank-major": rank r occupies elements
 * [r*n, (r+1)*n)).  Chunk c of a rank buffer is elements [c*C, (c+1)*C) with
 * C = n / P; the ring schedule requires P to divide n ("全归约 3：Ring——每步
 * 大小恒定", section "Run it": SIZE must be divisible by the rank count).
 *
 * The ring (same page, "Walkthrough"; also "Pallas TPU Distributed
 * Collectives 复习文档" section 0.1): data travels from rank r to its right
 * neighbour (r + 1) mod P, so rank r receives from its left neighbour
 * (r - 1 + P) mod P -- the "+P" keeps the dividend non-negative.
 *
 * Every step below is applied to all ranks "at once": the new chunk values of
 * a step are first computed for every rank from the state before the step and
 * only then stored, so no rank can observe another rank's write of the same
 * step.  This is the plain meaning of one round of the schedule.
 *
 * Return codes: 0 = ok, -1 = invalid arguments.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

/* left neighbour, never negative ("Walkthrough", and its edge-case table) */
static int left_of(int r, int P) { return (r - 1 + P) % P; }

/*
 * Reduce-scatter chunk for rank r at round s (s = 0 .. P-2).  On the ring
 * page ("全归约 3：Ring——每步大小恒定", Walkthrough) the chunk a rank adds
 * its own data into and the chunk its left neighbour sent are, at round s,
 * both the one numbered (r - s - 2) mod P: counting the step from 1, the
 * receiver's index is its rank minus the step minus one, and the sender's is
 * the sender's rank (one less) minus the step.  2P is added so the dividend
 * stays >= 0.
 */
static int rs_chunk(int r, int s, int P) { return (r - s - 2 + 2 * P) % P; }

/*
 * All-gather chunk for rank r at round t (t = 0 .. P-2).  The ring page leaves
 * the indices of its second phase unprinted (it only says each rank copies the
 * chunk its left neighbour sent into its own copy).  The reading used: at
 * round t rank r receives chunk (r - t - 1) mod P from its left neighbour and
 * stores it at the same chunk position.  This is the slot rule of
 * "Pallas TPU Distributed Collectives 复习文档" section 2.4 (a device forwards
 * slot (id - step) mod P to the same slot of its right neighbour), seen from
 * the receiving side.
 */
static int ag_chunk(int r, int t, int P) { return (r - t - 1 + P) % P; }

static int check_args(int P, size_t n)
{
    if (P < 1 || P > 64) return -1;
    if (n % (size_t)P != 0) return -1;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* ppermute: every rank sends its whole buffer to the right neighbour, so    */
/* rank r ends with what rank left(r) held ("Pallas TPU Distributed          */
/* Collectives 复习文档" section 1, the right-shift example).  Byte copy.     */
/* ------------------------------------------------------------------------ */
int oracle_ppermute(const void *src, void *dst, int P, size_t bytes_per_rank)
{
    if (P < 1 || P > 64 || src == dst) return -1;
    const uint8_t *s = (const uint8_t *)src;
    uint8_t *d = (uint8_t *)dst;
    for (int r = 0; r < P; ++r)
        memcpy(d + (size_t)r * bytes_per_rank,
               s + (size_t)left_of(r, P) * bytes_per_rank, bytes_per_rank);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Reduce-scatter, fp32 ("全归约 3", Walkthrough, first loop).               */
/*                                                                          */
/* state starts as a copy of src (the page works in place on a buffer that  */
/* holds the input).  At round s every rank r takes chunk c = rs_chunk(r,s) */
/* of its left neighbour (the partial sum that neighbour stored in round    */
/* s-1; at s = 0 simply the neighbour's input), adds its own input chunk c  */
/* to it, and stores the sum as its chunk c.  After P-1 rounds chunk r of   */
/* rank r holds the sum over all ranks.                                     */
/*                                                                          */
/* `rounds` (0 .. P-1) lets tests stop early and look at the state.         */
/* ------------------------------------------------------------------------ */
int oracle_reduce_scatter_f32(const float *src, float *state, int P, size_t n,
                              int rounds)
{
    if (check_args(P, n) || rounds < 0 || rounds > P - 1) return -1;
    const size_t C = n / (size_t)P;
    memmove(state, src, sizeof(float) * (size_t)P * n);
    float *tmp = (float *)malloc(sizeof(float) * (C ? C : 1) * (size_t)P);
    if (!tmp) return -1;
    for (int s = 0; s < rounds; ++s) {
        /* compute every rank's new chunk from the state before the round */
        for (int r = 0; r < P; ++r) {
            const int c = rs_chunk(r, s, P);
            const float *recv = state + (size_t)left_of(r, P) * n + (size_t)c * C;
            const float *own = src + (size_t)r * n + (size_t)c * C;
            for (size_t i = 0; i < C; ++i)
                tmp[(size_t)r * C + i] = own[i] + recv[i];
        }
        /* then store them */
        for (int r = 0; r < P; ++r) {
            const int c = rs_chunk(r, s, P);
            memcpy(state + (size_t)r * n + (size_t)c * C, tmp + (size_t)r * C,
                   sizeof(float) * C);
        }
    }
    free(tmp);
    return 0;
}

/* Reduce-scatter, int32.  Same schedule; additions wrap modulo 2^32
 * (two's complement), done in unsigned arithmetic so C has no overflow. */
int oracle_reduce_scatter_i32(const int32_t *src, int32_t *state, int P,
                              size_t n, int rounds)
{
    if (check_args(P, n) || rounds < 0 || rounds > P - 1) return -1;
    const size_t C = n / (size_t)P;
    memmove(state, src, sizeof(int32_t) * (size_t)P * n);
    uint32_t *tmp = (uint32_t *)malloc(sizeof(uint32_t) * (C ? C : 1) * (size_t)P);
    if (!tmp) return -1;
    for (int s = 0; s < rounds; ++s) {
        for (int r = 0; r < P; ++r) {
            const int c = rs_chunk(r, s, P);
            const int32_t *recv = state + (size_t)left_of(r, P) * n + (size_t)c * C;
            const int32_t *own = src + (size_t)r * n + (size_t)c * C;
            for (size_t i = 0; i < C; ++i)
                tmp[(size_t)r * C + i] = (uint32_t)own[i] + (uint32_t)recv[i];
        }
        for (int r = 0; r < P; ++r) {
            const int c = rs_chunk(r, s, P);
            memcpy(state + (size_t)r * n + (size_t)c * C, tmp + (size_t)r * C,
                   sizeof(int32_t) * C);
        }
    }
    free(tmp);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* All-gather ("全归约 3", Walkthrough, second phase; slot rule of           */
/* "Pallas TPU Distributed Collectives 复习文档" section 2).  A pure copy, so */
/* it works on raw elements of size esize.  On entry chunk r of rank r must  */
/* hold rank r's piece; at round t every rank r copies chunk ag_chunk(r,t)  */
/* of its left neighbour into the same chunk of its own buffer.             */
/* ------------------------------------------------------------------------ */
int oracle_all_gather(void *state, int P, size_t n, size_t esize, int rounds)
{
    if (check_args(P, n) || rounds < 0 || rounds > P - 1 || esize == 0) return -1;
    const size_t Cb = (n / (size_t)P) * esize;      /* chunk bytes */
    const size_t nb = n * esize;                    /* rank bytes */
    uint8_t *st = (uint8_t *)state;
    uint8_t *tmp = (uint8_t *)malloc((Cb ? Cb : 1) * (size_t)P);
    if (!tmp) return -1;
    for (int t = 0; t < rounds; ++t) {
        for (int r = 0; r < P; ++r) {
            const int c = ag_chunk(r, t, P);
            memcpy(tmp + (size_t)r * Cb, st + (size_t)left_of(r, P) * nb + (size_t)c * Cb, Cb);
        }
        for (int r = 0; r < P; ++r) {
            const int c = ag_chunk(r, t, P);
            memcpy(st + (size_t)r * nb + (size_t)c * Cb, tmp + (size_t)r * Cb, Cb);
        }
    }
    free(tmp);
    return 0;
}

/* Place each rank's compact piece (C elements) at chunk r of its own buffer,
 * the first action of the all-gather examples ("Pallas TPU Distributed
 * Collectives 复习文档" section 2.3, and the all-gather kernel of "TPU 与分布式
 * 通信原语"). */
int oracle_all_gather_place(const void *pieces, void *state, int P, size_t n,
                            size_t esize)
{
    if (check_args(P, n) || esize == 0) return -1;
    const size_t Cb = (n / (size_t)P) * esize;
    const size_t nb = n * esize;
    for (int r = 0; r < P; ++r)
        memcpy((uint8_t *)state + (size_t)r * nb + (size_t)r * Cb,
               (const uint8_t *)pieces + (size_t)r * Cb, Cb);
    return 0;
}

/* All-reduce = reduce-scatter (P-1 rounds) then all-gather (P-1 rounds) on
 * the same buffers ("全归约 3", "The idea"). */
int oracle_all_reduce_f32(const float *src, float *state, int P, size_t n)
{
    if (oracle_reduce_scatter_f32(src, state, P, n, P - 1)) return -1;
    return oracle_all_gather(state, P, n, sizeof(float), P - 1);
}

int oracle_all_reduce_i32(const int32_t *src, int32_t *state, int P, size_t n)
{
    if (oracle_reduce_scatter_i32(src, state, P, n, P - 1)) return -1;
    return oracle_all_gather(state, P, n, sizeof(int32_t), P - 1);
}

/* ------------------------------------------------------------------------ */
/* bfloat16.                                                                 */
/*                                                                          */
/* bf16 is the upper 16 bits of an IEEE-754 binary32.  Conversion from fp32 */
/* rounds to nearest, ties to even, on the 16 dropped bits: add 0x7FFF plus  */
/* the lowest kept bit, then truncate.  NaN stays NaN (quiet bit forced).   */
/* ------------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_bf16_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);        /* quiet NaN */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void oracle_bf16_from_f32_array(const float *x, uint16_t *y, size_t m)
{
    for (size_t i = 0; i < m; ++i) y[i] = oracle_bf16_from_f32(x[i]);
}

/*
 * Reduce-scatter on bf16 data with an fp32 carry.  The pages keep partial
 * sums in the buffer's own type; for bf16 inputs with "fp32 accumulation,
 * bf16 output" the reading taken is: partial sums travel between ranks in
 * fp32 (the carry), and only the owner's final sum is rounded once to bf16.
 *
 *   carry  : P*n fp32, starts as the fp32 value of every input element;
 *   round s: carry[r][c] = carry_before[left][c] + f32(src[r][c]);
 *   last round (s = P-2) additionally sets dst[r][r] = bf16(carry[r][r]).
 * dst starts as a copy of src.
 */
int oracle_reduce_scatter_bf16(const uint16_t *src, uint16_t *dst, float *carry,
                               int P, size_t n, int rounds)
{
    if (check_args(P, n) || rounds < 0 || rounds > P - 1) return -1;
    const size_t C = n / (size_t)P;
    memmove(dst, src, sizeof(uint16_t) * (size_t)P * n);
    for (size_t i = 0; i < (size_t)P * n; ++i) carry[i] = bf16_to_f32(src[i]);
    float *tmp = (float *)malloc(sizeof(float) * (C ? C : 1) * (size_t)P);
    if (!tmp) return -1;
    for (int s = 0; s < rounds; ++s) {
        for (int r = 0; r < P; ++r) {
            const int c = rs_chunk(r, s, P);
            const float *recv = carry + (size_t)left_of(r, P) * n + (size_t)c * C;
            const uint16_t *own = src + (size_t)r * n + (size_t)c * C;
            for (size_t i = 0; i < C; ++i)
                tmp[(size_t)r * C + i] = bf16_to_f32(own[i]) + recv[i];
        }
        for (int r = 0; r < P; ++r) {
            const int c = rs_chunk(r, s, P);
            memcpy(carry + (size_t)r * n + (size_t)c * C, tmp + (size_t)r * C,
                   sizeof(float) * C);
            if (s == P - 2)      /* c == r here: the owner's last round */
                for (size_t i = 0; i < C; ++i)
                    dst[(size_t)r * n + (size_t)c * C + i] =
                        oracle_bf16_from_f32(tmp[(size_t)r * C + i]);
        }
    }
    free(tmp);
    return 0;
}

int oracle_all_reduce_bf16(const uint16_t *src, uint16_t *dst, float *carry,
                           int P, size_t n)
{
    if (oracle_reduce_scatter_bf16(src, dst, carry, P, n, P - 1)) return -1;
    return oracle_all_gather(dst, P, n, sizeof(uint16_t), P - 1);
}

/* ------------------------------------------------------------------------ */
/* Bidirectional reduce-scatter ("Pallas TPU Distributed Collectives 复习文档" */
/* section 4, lax.psum_scatter, and its P = 4 walk-through in 4.6).          */
/*                                                                          */
/* Every chunk (the page's "block") is split into a top half, which travels  */
/* to the LEFT neighbour, and a bottom half, which travels to the RIGHT one. */
/* Device d first hands the halves of its own block d to its neighbours.    */
/* At step s = 0 .. P-2 it takes the top half it received from its right    */
/* neighbour, adds its own contribution to block (d + s + 1) mod P, and     */
/* passes the sum on to the left; likewise the bottom half received from    */
/* the left neighbour gets its contribution to block (d - s - 1) mod P and  */
/* goes on to the right.  At the last step (s = P - 1) the halves that      */
/* arrive belong to block d and are complete: they are kept, nothing more   */
/* is added.  So the top half of block b is summed owner first,             */
/*     ((x_b + x_{b-1}) + x_{b-2}) + ... + x_{b+1},                         */
/* and the bottom half ((x_b + x_{b+1}) + x_{b+2}) + ... + x_{b-1}.          */
/*                                                                          */
/* Reading for the split of a chunk of C elements (the page's blocks have   */
/* an even number of rows): the top half is the first C - C/2 elements.     */
/*                                                                          */
/* `state` (P*n, rank-major) starts as a copy of src.  The sum a device     */
/* computes at step s is stored at the half it belongs to: the top half of  */
/* chunk (d + s + 1) mod P and the bottom half of chunk (d - s - 1) mod P   */
/* of device d's buffer; the last step stores the complete block d in chunk */
/* d.  `steps` (0 .. P) lets tests stop early and look at the state.        */
/* ------------------------------------------------------------------------ */
static size_t bidir_top_len(size_t C) { return C - C / 2; }
static int mod_p(int x, int P) { return ((x % P) + P) % P; }

int oracle_reduce_scatter_bidir_f32(const float *src, float *state, int P, size_t n,
                                    int steps)
{
    if (check_args(P, n) || steps < 0 || steps > P) return -1;
    const size_t C = n / (size_t)P, h = bidir_top_len(C), hb = C - h;
    memmove(state, src, sizeof(float) * (size_t)P * n);
    /* the half each device passes on next: top to the left, bottom to the right */
    float *top = (float *)malloc(sizeof(float) * (h ? h : 1) * (size_t)P);
    float *bot = (float *)malloc(sizeof(float) * (hb ? hb : 1) * (size_t)P);
    float *ntop = (float *)malloc(sizeof(float) * (h ? h : 1) * (size_t)P);
    float *nbot = (float *)malloc(sizeof(float) * (hb ? hb : 1) * (size_t)P);
    if (!top || !bot || !ntop || !nbot) { free(top); free(bot); free(ntop); free(nbot); return -1; }
    for (int d = 0; d < P; ++d) {
        const float *own = src + (size_t)d * n + (size_t)d * C;
        memcpy(top + (size_t)d * h, own, sizeof(float) * h);
        memcpy(bot + (size_t)d * hb, own + h, sizeof(float) * hb);
    }
    for (int s = 0; s < steps; ++s) {
        const int last = (s == P - 1);
        for (int d = 0; d < P; ++d) {
            const float *from_right = top + (size_t)mod_p(d + 1, P) * h;
            const float *from_left = bot + (size_t)mod_p(d - 1, P) * hb;
            const float *xt = src + (size_t)d * n + (size_t)mod_p(d + s + 1, P) * C;
            const float *xb = src + (size_t)d * n + (size_t)mod_p(d - s - 1, P) * C + h;
            for (size_t i = 0; i < h; ++i)
                ntop[(size_t)d * h + i] = last ? from_right[i] : from_right[i] + xt[i];
            for (size_t i = 0; i < hb; ++i)
                nbot[(size_t)d * hb + i] = last ? from_left[i] : from_left[i] + xb[i];
        }
        for (int d = 0; d < P; ++d) {
            const int ct = last ? d : mod_p(d + s + 1, P);
            const int cb = last ? d : mod_p(d - s - 1, P);
            memcpy(state + (size_t)d * n + (size_t)ct * C, ntop + (size_t)d * h, sizeof(float) * h);
            memcpy(state + (size_t)d * n + (size_t)cb * C + h, nbot + (size_t)d * hb, sizeof(float) * hb);
        }
        float *t = top; top = ntop; ntop = t;
        t = bot; bot = nbot; nbot = t;
    }
    free(top); free(bot); free(ntop); free(nbot);
    return 0;
}

/* The same schedule on int32; additions wrap modulo 2^32. */
int oracle_reduce_scatter_bidir_i32(const int32_t *src, int32_t *state, int P, size_t n,
                                    int steps)
{
    if (check_args(P, n) || steps < 0 || steps > P) return -1;
    const size_t C = n / (size_t)P, h = bidir_top_len(C), hb = C - h;
    memmove(state, src, sizeof(int32_t) * (size_t)P * n);
    uint32_t *top = (uint32_t *)malloc(sizeof(uint32_t) * (h ? h : 1) * (size_t)P);
    uint32_t *bot = (uint32_t *)malloc(sizeof(uint32_t) * (hb ? hb : 1) * (size_t)P);
    uint32_t *ntop = (uint32_t *)malloc(sizeof(uint32_t) * (h ? h : 1) * (size_t)P);
    uint32_t *nbot = (uint32_t *)malloc(sizeof(uint32_t) * (hb ? hb : 1) * (size_t)P);
    if (!top || !bot || !ntop || !nbot) { free(top); free(bot); free(ntop); free(nbot); return -1; }
    for (int d = 0; d < P; ++d) {
        const int32_t *own = src + (size_t)d * n + (size_t)d * C;
        memcpy(top + (size_t)d * h, own, sizeof(int32_t) * h);
        memcpy(bot + (size_t)d * hb, own + h, sizeof(int32_t) * hb);
    }
    for (int s = 0; s < steps; ++s) {
        const int last = (s == P - 1);
        for (int d = 0; d < P; ++d) {
            const uint32_t *from_right = top + (size_t)mod_p(d + 1, P) * h;
            const uint32_t *from_left = bot + (size_t)mod_p(d - 1, P) * hb;
            const int32_t *xt = src + (size_t)d * n + (size_t)mod_p(d + s + 1, P) * C;
            const int32_t *xb = src + (size_t)d * n + (size_t)mod_p(d - s - 1, P) * C + h;
            for (size_t i = 0; i < h; ++i)
                ntop[(size_t)d * h + i] = last ? from_right[i] : from_right[i] + (uint32_t)xt[i];
            for (size_t i = 0; i < hb; ++i)
                nbot[(size_t)d * hb + i] = last ? from_left[i] : from_left[i] + (uint32_t)xb[i];
        }
        for (int d = 0; d < P; ++d) {
            const int ct = last ? d : mod_p(d + s + 1, P);
            const int cb = last ? d : mod_p(d - s - 1, P);
            memcpy(state + (size_t)d * n + (size_t)ct * C, ntop + (size_t)d * h, sizeof(int32_t) * h);
            memcpy(state + (size_t)d * n + (size_t)cb * C + h, nbot + (size_t)d * hb, sizeof(int32_t) * hb);
        }
        uint32_t *t = top; top = ntop; ntop = t;
        t = bot; bot = nbot; nbot = t;
    }
    free(top); free(bot); free(ntop); free(nbot);
    return 0;
}

/*
 * bf16 inputs with fp32 partial sums (the reading used for the one-way ring
 * as well): the halves travel in fp32, `carry` (P*n) receives each step's
 * sums at the same positions as `state` in the fp32 version, and only the
 * complete block is rounded once to bf16, at the last step, into dst[d][d].
 * dst starts as a copy of src.
 */
int oracle_reduce_scatter_bidir_bf16(const uint16_t *src, uint16_t *dst, float *carry,
                                     int P, size_t n, int steps)
{
    if (check_args(P, n) || steps < 0 || steps > P) return -1;
    const size_t C = n / (size_t)P, h = bidir_top_len(C), hb = C - h;
    memmove(dst, src, sizeof(uint16_t) * (size_t)P * n);
    for (size_t i = 0; i < (size_t)P * n; ++i) carry[i] = bf16_to_f32(src[i]);
    float *top = (float *)malloc(sizeof(float) * (h ? h : 1) * (size_t)P);
    float *bot = (float *)malloc(sizeof(float) * (hb ? hb : 1) * (size_t)P);
    float *ntop = (float *)malloc(sizeof(float) * (h ? h : 1) * (size_t)P);
    float *nbot = (float *)malloc(sizeof(float) * (hb ? hb : 1) * (size_t)P);
    if (!top || !bot || !ntop || !nbot) { free(top); free(bot); free(ntop); free(nbot); return -1; }
    for (int d = 0; d < P; ++d) {
        const uint16_t *own = src + (size_t)d * n + (size_t)d * C;
        for (size_t i = 0; i < h; ++i) top[(size_t)d * h + i] = bf16_to_f32(own[i]);
        for (size_t i = 0; i < hb; ++i) bot[(size_t)d * hb + i] = bf16_to_f32(own[h + i]);
    }
    for (int s = 0; s < steps; ++s) {
        const int last = (s == P - 1);
        for (int d = 0; d < P; ++d) {
            const float *from_right = top + (size_t)mod_p(d + 1, P) * h;
            const float *from_left = bot + (size_t)mod_p(d - 1, P) * hb;
            const uint16_t *xt = src + (size_t)d * n + (size_t)mod_p(d + s + 1, P) * C;
            const uint16_t *xb = src + (size_t)d * n + (size_t)mod_p(d - s - 1, P) * C + h;
            for (size_t i = 0; i < h; ++i)
                ntop[(size_t)d * h + i] = last ? from_right[i] : from_right[i] + bf16_to_f32(xt[i]);
            for (size_t i = 0; i < hb; ++i)
                nbot[(size_t)d * hb + i] = last ? from_left[i] : from_left[i] + bf16_to_f32(xb[i]);
        }
        for (int d = 0; d < P; ++d) {
            const int ct = last ? d : mod_p(d + s + 1, P);
            const int cb = last ? d : mod_p(d - s - 1, P);
            memcpy(carry + (size_t)d * n + (size_t)ct * C, ntop + (size_t)d * h, sizeof(float) * h);
            memcpy(carry + (size_t)d * n + (size_t)cb * C + h, nbot + (size_t)d * hb, sizeof(float) * hb);
            if (last) {
                uint16_t *o = dst + (size_t)d * n + (size_t)d * C;
                for (size_t i = 0; i < h; ++i) o[i] = oracle_bf16_from_f32(ntop[(size_t)d * h + i]);
                for (size_t i = 0; i < hb; ++i) o[h + i] = oracle_bf16_from_f32(nbot[(size_t)d * hb + i]);
            }
        }
        float *t = top; top = ntop; ntop = t;
        t = bot; bot = nbot; nbot = t;
    }
    free(top); free(bot); free(ntop); free(nbot);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Circulating-input psum ("Pallas TPU Distributed Collectives 复习文档",     */
/* section 3, lax.psum, and its walk-through table in 3.5).                 */
/*                                                                          */
/* Every device's whole input travels once around the ring to the right.   */
/* Each device has two receive slots (the page's hbm_buf[0] / hbm_buf[1])   */
/* and an accumulator that starts at zero.  First every device sends its    */
/* input into slot 0 of its right neighbour.  At step s = 0 .. P-1 a device */
/* adds what is in its slot s % 2 to its accumulator and forwards it to     */
/* slot (s + 1) % 2 of its right neighbour.  So device d adds x_{d-1},      */
/* x_{d-2}, ..., and last its own x_d, which comes back after P hops:       */
/*     out[d] = ((((0 + x_{d-1}) + x_{d-2}) + ...) + x_d.                   */
/* The page forwards at the last step too (the item has then been          */
/* everywhere; it changes only the slots, as its table shows).              */
/*                                                                          */
/* `slots` (2*P*n, device-major, slot-major) and `acc` (P*n) hold the state */
/* after `steps` steps (0 .. P); a slot never written holds 0.              */
/* ------------------------------------------------------------------------ */
int oracle_psum_circ_f32(const float *src, float *acc, float *slots, int P, size_t n, int steps)
{
    if (P < 1 || P > 64 || steps < 0 || steps > P) return -1;
    float *item = (float *)malloc(sizeof(float) * (n ? n : 1) * (size_t)P);
    if (!item) return -1;
    memset(acc, 0, sizeof(float) * (size_t)P * n);
    memset(slots, 0, sizeof(float) * 2 * (size_t)P * n);
    for (int d = 0; d < P; ++d)          /* the first send: input -> right neighbour's slot 0 */
        memcpy(slots + ((size_t)((d + 1) % P) * 2 + 0) * n, src + (size_t)d * n, sizeof(float) * n);
    for (int s = 0; s < steps; ++s) {
        const int w = s % 2;
        for (int d = 0; d < P; ++d) {    /* read every working slot first */
            const float *in = slots + ((size_t)d * 2 + w) * n;
            memcpy(item + (size_t)d * n, in, sizeof(float) * n);
            for (size_t i = 0; i < n; ++i) acc[(size_t)d * n + i] += in[i];
        }
        for (int d = 0; d < P; ++d)      /* then forward to the right neighbour's other slot */
            memcpy(slots + ((size_t)((d + 1) % P) * 2 + (1 - w)) * n, item + (size_t)d * n,
                   sizeof(float) * n);
    }
    free(item);
    return 0;
}

/* The same on int32 (wrapping adds). */
int oracle_psum_circ_i32(const int32_t *src, int32_t *acc, int32_t *slots, int P, size_t n, int steps)
{
    if (P < 1 || P > 64 || steps < 0 || steps > P) return -1;
    int32_t *item = (int32_t *)malloc(sizeof(int32_t) * (n ? n : 1) * (size_t)P);
    if (!item) return -1;
    memset(acc, 0, sizeof(int32_t) * (size_t)P * n);
    memset(slots, 0, sizeof(int32_t) * 2 * (size_t)P * n);
    for (int d = 0; d < P; ++d)
        memcpy(slots + ((size_t)((d + 1) % P) * 2 + 0) * n, src + (size_t)d * n, sizeof(int32_t) * n);
    for (int s = 0; s < steps; ++s) {
        const int w = s % 2;
        for (int d = 0; d < P; ++d) {
            const int32_t *in = slots + ((size_t)d * 2 + w) * n;
            memcpy(item + (size_t)d * n, in, sizeof(int32_t) * n);
            for (size_t i = 0; i < n; ++i)
                acc[(size_t)d * n + i] = (int32_t)((uint32_t)acc[(size_t)d * n + i] + (uint32_t)in[i]);
        }
        for (int d = 0; d < P; ++d)
            memcpy(slots + ((size_t)((d + 1) % P) * 2 + (1 - w)) * n, item + (size_t)d * n,
                   sizeof(int32_t) * n);
    }
    free(item);
    return 0;
}

/* bf16 inputs circulate unchanged; the accumulator is fp32 and the result
 * is rounded once to bf16 (the reading used for every bf16 sum here). */
int oracle_psum_circ_bf16(const uint16_t *src, uint16_t *dst, int P, size_t n)
{
    if (P < 1 || P > 64) return -1;
    float *acc = (float *)calloc((n ? n : 1) * (size_t)P, sizeof(float));
    if (!acc) return -1;
    for (int d = 0; d < P; ++d)
        for (int s = 0; s < P; ++s) {          /* item of step s: x_{(d - s - 1) mod P} */
            const uint16_t *in = src + (size_t)(((d - s - 1) % P + P) % P) * n;
            for (size_t i = 0; i < n; ++i) acc[(size_t)d * n + i] += bf16_to_f32(in[i]);
        }
    for (size_t i = 0; i < (size_t)P * n; ++i) dst[i] = oracle_bf16_from_f32(acc[i]);
    free(acc);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Plain definitions used as references for tolerance checks.               */
/* Sum over ranks in rank order 0..P-1, in fp64, and the sum of magnitudes  */
/* (the denominator of the componentwise error bound of recursive sums).    */
/* ------------------------------------------------------------------------ */
int oracle_rank_sum_f64_f32(const float *src, int P, size_t n, double *sum,
                            double *abssum)
{
    if (P < 1) return -1;
    for (size_t i = 0; i < n; ++i) {
        double a = 0.0, m = 0.0;
        for (int q = 0; q < P; ++q) {
            const double x = (double)src[(size_t)q * n + i];
            a += x;
            m += fabs(x);
        }
        sum[i] = a;
        if (abssum) abssum[i] = m;
    }
    return 0;
}

int oracle_rank_sum_f64_bf16(const uint16_t *src, int P, size_t n, double *sum,
                             double *abssum)
{
    if (P < 1) return -1;
    for (size_t i = 0; i < n; ++i) {
        double a = 0.0, m = 0.0;
        for (int q = 0; q < P; ++q) {
            const double x = (double)bf16_to_f32(src[(size_t)q * n + i]);
            a += x;
            m += fabs(x);
        }
        sum[i] = a;
        if (abssum) abssum[i] = m;
    }
    return 0;
}

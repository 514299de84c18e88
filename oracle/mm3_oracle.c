/*
 * mm3_oracle.c -- plain CPU oracle for the block-scored paged index top-k.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call this file:
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load it.  It shares no source, header, table or helper with the HIP
 * library; it is written straight from the pages' statement of the problem:
 *
 *   "vllm.models.minimax_m3.amd.ops.index_topk", module docstring: every
 *   index query scores each 128-token block of a paged, shared index-K
 *   cache (one page == one block), the score is the maximum over the block,
 *   and per query token the top-k blocks plus the forced init/local blocks
 *   are selected; functions minimax_m3_index_decode / minimax_m3_index_topk
 *   docstrings: 0-indexed logical block ids, -1 padding.
 *
 *   "vllm.models.minimax_m3.amd.indexer_nvfp4", module docstring: NVFP4
 *   index keys score as e4m3_rn_satfinite(e2m1 * scale).
 *
 * Arithmetic is fp64 unless the pages fix it: each dot product is summed in
 * double in ascending d, the block maximum is taken in double, and only the
 * final sm_scale * max is rounded once to the fp32 score the pages' score
 * tensors hold (torch.float32 in minimax_m3_index_decode / _new_score).
 *
 * Readings taken where the pages are silent:
 *   - the Q rows of request r sit at positions seq_len[r]-Q+j, j<Q;
 *   - ragged batches (minimax_m3_index_score / minimax_m3_index_topk take
 *     cu_seqlens_q and prefix_lens): request r owns rows
 *     [cu_seqlens_q[r], cu_seqlens_q[r+1]) and its row j sits at position
 *     prefix_lens[r] + j; without prefix_lens (the NVFP4 prefill scorer of
 *     page "indexer_nvfp4" takes only cu_seqlens_q and seq_lens) the rows are
 *     the request's last tokens, seq_lens[r] - n_r + j;
 *   - a row at position pos sees blocks b <= pos/128, and in block b the
 *     tokens 128b+s <= pos;
 *   - forced blocks take slots inside topk; init and local overlap is
 *     de-duplicated; the remaining slots go to the best other visible blocks
 *     by (score descending, id ascending);
 *   - a row's ids are written in ascending order, then -1 up to topk;
 *   - NVFP4 key layout: nibbles [pages][128][64], element 2i in the low
 *     nibble of byte i, element 2i+1 in the high nibble; scales
 *     [pages][128][8], scale g covers d in [16g, 16g+16).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BLOCK 128
#define ORC_DIM 128

/* ---------------------------------------------------------------- codecs */

/* bfloat16 bit pattern -> double (bf16 is the top half of an IEEE binary32) */
static double orc_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* FP4 E2M1 (OCP MX): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent 0 is subnormal: 0.m * 2^0. Magnitudes 0,0.5,1,1.5,2,3,4,6. */
double oracle_e2m1_value(int nib)
{
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* FP8 E4M3FN (OCP): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa; exponent 0 subnormal (m/8 * 2^-6); no infinities; S.1111.111 NaN. */
double oracle_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp(m / 8.0, -6);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round x to the E4M3FN grid: nearest representable finite value, ties to the
 * even code (even mantissa), and saturation to +-448 instead of overflow.
 * Written as a search over the 127 non-negative finite codes so that it is
 * checkable by eye; codes are ordered by value. */
double oracle_e4m3_rn_satfinite(double x)
{
    double a = fabs(x), best = 0.0, bestd = INFINITY;
    int bestc = 0;
    if (a >= 448.0) {
        best = 448.0;
    } else {
        for (int c = 0; c <= 126; ++c) {
            double v = oracle_e4m3_value(c);
            double d = fabs(v - a);
            if (d < bestd || (d == bestd && (c & 1) == 0 && (bestc & 1) == 1)) {
                bestd = d;
                best = v;
                bestc = c;
            }
        }
    }
    return signbit(x) ? -best : best;
}

/* One NVFP4 key element: e4m3_rn_satfinite(e2m1(nib) * e4m3(scale)).
 * The product of a 2-significant-bit and a 4-significant-bit value is exact
 * in double, so the only rounding is the E4M3 one. */
double oracle_nvfp4_element(int nib, int scale_byte)
{
    return oracle_e4m3_rn_satfinite(oracle_e2m1_value(nib) *
                                    oracle_e4m3_value(scale_byte));
}

/* ---------------------------------------------------------- row mapping */

/*
 * Request and position of row t.  Uniform batches (cu == NULL): request
 * r = t / Q owns rows [rQ, rQ+Q) and its row j sits at seq_lens[r] - Q + j.
 * Ragged batches: r is the request with cu[r] <= t < cu[r+1] (found by a
 * plain scan), j = t - cu[r], and the position is prefix[r] + j, or
 * seq_lens[r] - (cu[r+1] - cu[r]) + j without prefix.  Returns 0, or -1 when
 * t is outside the batch.
 */
static int orc_row(int64_t t, const int32_t* seq_lens, int num_reqs,
                   int query_len, const int32_t* cu, const int32_t* prefix,
                   int* r_out, int64_t* pos_out)
{
    if (!cu) {
        if (t < 0 || t >= (int64_t)num_reqs * query_len)
            return -1;
        int r = (int)(t / query_len);
        *r_out = r;
        *pos_out = (int64_t)seq_lens[r] - query_len + (t % query_len);
        return 0;
    }
    for (int r = 0; r < num_reqs; ++r) {
        if (cu[r] <= t && t < cu[r + 1]) {
            int64_t j = t - cu[r];
            int64_t n = (int64_t)cu[r + 1] - cu[r];
            *r_out = r;
            *pos_out = prefix ? (int64_t)prefix[r] + j
                              : (int64_t)seq_lens[r] - n + j;
            return 0;
        }
    }
    return -1;
}

static int64_t orc_total_rows(int num_reqs, int query_len, const int32_t* cu)
{
    return cu ? (int64_t)cu[num_reqs] : (int64_t)num_reqs * query_len;
}

/* ------------------------------------------------------------ block scores */

typedef struct {
    double v[16][256];
    int ready;
} orc_fp4_table;

static void orc_fp4_table_init(orc_fp4_table* t)
{
    for (int n = 0; n < 16; ++n)
        for (int s = 0; s < 256; ++s)
            t->v[n][s] = oracle_nvfp4_element(n, s);
    t->ready = 1;
}

/* Key element d of token tok of page `page`, as a double. */
static double orc_key(int kfmt, const void* kdata, const uint8_t* kscales,
                      const orc_fp4_table* t, int64_t page, int tok, int d)
{
    if (kfmt == 0) {
        const uint16_t* k = (const uint16_t*)kdata;
        return orc_bf16(k[(page * ORC_BLOCK + tok) * ORC_DIM + d]);
    } else {
        const uint8_t* nb = (const uint8_t*)kdata;
        uint8_t byte = nb[(page * ORC_BLOCK + tok) * (ORC_DIM / 2) + d / 2];
        int nib = (d & 1) ? (byte >> 4) : (byte & 15);
        uint8_t sc = kscales[(page * ORC_BLOCK + tok) * (ORC_DIM / 16) + d / 16];
        return t->v[nib][sc];
    }
}

/*
 * Block scores.  For every requested row t (all rows when rows == NULL):
 *   request r and position pos as orc_row gives them; rows with pos < 0 see
 *   nothing and are skipped.  For head h and visible block b <= pos/128:
 *     page = block_table[r][b], n = min(128, pos - 128 b + 1),
 *     score[h][t][b] = fl32( sm_scale * max_{s<n} sum_d q[t][h][d] k[page][s][d] ).
 * Blocks past pos/128 are not written.  scores64 (NULL allowed, same strides)
 * receives the same value before its one rounding to fp32: two blocks whose
 * scores64 are equal hold keys with the same largest dot product, a true
 * tie, while equal fp32 scores may also come from distinct values that round
 * alike.
 * Returns 0, or -1 on a bad argument (page id out of range, ...).
 */
int oracle_block_scores(const uint16_t* q, int64_t q_tok_stride,
                        int64_t q_head_stride, int heads, int kfmt,
                        const void* kdata, const uint8_t* kscales,
                        int64_t num_pages, const int32_t* block_table,
                        int64_t bt_row_stride, const int32_t* seq_lens,
                        int num_reqs, int query_len,
                        const int32_t* cu_seqlens_q, const int32_t* prefix_lens,
                        float sm_scale, float* scores, double* scores64,
                        int64_t s_head_stride, int64_t s_row_stride,
                        const int64_t* rows, int64_t num_rows)
{
    static orc_fp4_table table;
    if (kfmt == 1 && !table.ready)
        orc_fp4_table_init(&table);
    if ((!cu_seqlens_q && query_len <= 0) || heads <= 0)
        return -1;
    int64_t total = orc_total_rows(num_reqs, query_len, cu_seqlens_q);
    int64_t n = rows ? num_rows : total;
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = rows ? rows[i] : i;
        int r;
        int64_t pos;
        if (orc_row(t, seq_lens, num_reqs, query_len, cu_seqlens_q,
                    prefix_lens, &r, &pos) != 0)
            return -1;
        if (pos < 0)
            continue;
        int64_t nv = pos / ORC_BLOCK + 1;
        for (int h = 0; h < heads; ++h) {
            const uint16_t* qr = q + t * q_tok_stride + h * q_head_stride;
            for (int64_t b = 0; b < nv; ++b) {
                int64_t page = block_table[r * bt_row_stride + b];
                if (page < 0 || page >= num_pages)
                    return -1;
                int64_t cnt = pos - ORC_BLOCK * b + 1;
                if (cnt > ORC_BLOCK)
                    cnt = ORC_BLOCK;
                double best = -INFINITY;
                for (int s = 0; s < cnt; ++s) {
                    double dot = 0.0;
                    for (int d = 0; d < ORC_DIM; ++d)
                        dot += orc_bf16(qr[d]) *
                               orc_key(kfmt, kdata, kscales, &table, page, s, d);
                    if (dot > best)
                        best = dot;
                }
                double v = (double)sm_scale * best;
                scores[h * s_head_stride + t * s_row_stride + b] = (float)v;
                if (scores64)
                    scores64[h * s_head_stride + t * s_row_stride + b] = v;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ top-k */

typedef struct {
    float score;
    int32_t id;
} orc_cand;

/* (score descending, id ascending); -0 and +0 compare equal as floats */
static int orc_cand_cmp(const void* pa, const void* pb)
{
    const orc_cand* a = (const orc_cand*)pa;
    const orc_cand* b = (const orc_cand*)pb;
    if (a->score > b->score)
        return -1;
    if (a->score < b->score)
        return 1;
    return (a->id > b->id) - (a->id < b->id);
}

/*
 * Per (head, row) selection from a score tensor laid out as above.  With
 * nv = pos/128 + 1 visible blocks:
 *   F = [0, min(I, nv)) U [max(0, nv - L), nv)            (forced, pinned)
 *   nv <= topk : S = [0, nv)
 *   otherwise  : S = F plus the first topk - |F| blocks of [0, nv) \ F in
 *                (score descending, id ascending) order
 * out[h][t][:] = S in ascending order, then -1 up to topk.  Rows with
 * pos < 0 are all -1.  Returns 0, or -1 on bad arguments.
 */
int oracle_topk(const float* scores, int64_t s_head_stride,
                int64_t s_row_stride, int heads, const int32_t* seq_lens,
                int num_reqs, int query_len, const int32_t* cu_seqlens_q,
                const int32_t* prefix_lens, int topk, int init_blocks,
                int local_blocks, int32_t* out, int64_t o_head_stride,
                int64_t o_row_stride, const int64_t* rows, int64_t num_rows)
{
    if (topk <= 0 || init_blocks < 0 || local_blocks < 0 ||
        init_blocks + local_blocks > topk || (!cu_seqlens_q && query_len <= 0))
        return -1;
    int64_t total = orc_total_rows(num_reqs, query_len, cu_seqlens_q);
    int64_t n = rows ? num_rows : total;
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = rows ? rows[i] : i;
        int r;
        int64_t pos;
        if (orc_row(t, seq_lens, num_reqs, query_len, cu_seqlens_q,
                    prefix_lens, &r, &pos) != 0)
            return -1;
        (void)r;
        int64_t nv = pos < 0 ? 0 : pos / ORC_BLOCK + 1;
        char* sel = (char*)calloc(nv > 0 ? (size_t)nv : 1, 1);
        orc_cand* c = (orc_cand*)malloc((nv > 0 ? (size_t)nv : 1) * sizeof *c);
        if (!sel || !c) {
            free(sel);
            free(c);
            return -1;
        }
        for (int h = 0; h < heads; ++h) {
            const float* srow = scores + h * s_head_stride + t * s_row_stride;
            memset(sel, 0, nv > 0 ? (size_t)nv : 1);
            if (nv <= topk) {
                for (int64_t b = 0; b < nv; ++b)
                    sel[b] = 1;
            } else {
                int64_t nforced = 0, nc = 0;
                for (int64_t b = 0; b < nv; ++b) {
                    int forced = (b < init_blocks) || (b >= nv - local_blocks);
                    if (forced) {
                        sel[b] = 1;
                        ++nforced;
                    } else {
                        c[nc].score = srow[b];
                        c[nc].id = (int32_t)b;
                        ++nc;
                    }
                }
                qsort(c, (size_t)nc, sizeof *c, orc_cand_cmp);
                for (int64_t k = 0; k < topk - nforced && k < nc; ++k)
                    sel[c[k].id] = 1;
            }
            int32_t* orow = out + h * o_head_stride + t * o_row_stride;
            int w = 0;
            for (int64_t b = 0; b < nv; ++b)
                if (sel[b])
                    orow[w++] = (int32_t)b;
            while (w < topk)
                orow[w++] = -1;
        }
        free(sel);
        free(c);
    }
    return 0;
}

/* ------------------------------------------------------ sparse block table */

/*
 * Sparse block table for one index head, from selected ids (the optional
 * table arguments of minimax_m3_index_decode): the P attention pages of
 * sparse block b are entries [b*stride, b*stride + P) of the request's
 * attention block table.  For row t with selected ids b_0 < b_1 < ... :
 *   sparse[t][j*P + i] = abt[r][b_j * stride + i], -1 for unused slots,
 *   ctx_len[t] = sum_j min(128, pos - 128 b_j + 1)   (0 when pos < 0).
 */
int oracle_sparse_block_table(const int32_t* topk_idx, int64_t o_row_stride,
                              int topk, const int32_t* seq_lens, int num_reqs,
                              int query_len, const int32_t* cu_seqlens_q,
                              const int32_t* prefix_lens, const int32_t* abt,
                              int64_t abt_row_stride, int pages_per_block,
                              int block_page_stride, int32_t* sparse,
                              int64_t st_row_stride, int32_t* ctx_lens)
{
    if (topk <= 0 || (!cu_seqlens_q && query_len <= 0) || pages_per_block <= 0)
        return -1;
    int64_t total = orc_total_rows(num_reqs, query_len, cu_seqlens_q);
    for (int64_t t = 0; t < total; ++t) {
        int r;
        int64_t pos;
        if (orc_row(t, seq_lens, num_reqs, query_len, cu_seqlens_q,
                    prefix_lens, &r, &pos) != 0)
            return -1;
        int64_t len = 0;
        for (int k = 0; k < topk; ++k) {
            int32_t b = topk_idx[t * o_row_stride + k];
            for (int i = 0; i < pages_per_block; ++i)
                sparse[t * st_row_stride + (int64_t)k * pages_per_block + i] =
                    b < 0 ? -1
                          : abt[r * abt_row_stride +
                                (int64_t)b * block_page_stride + i];
            if (b >= 0 && pos >= 0) {
                int64_t cnt = pos - (int64_t)ORC_BLOCK * b + 1;
                if (cnt > ORC_BLOCK)
                    cnt = ORC_BLOCK;
                if (cnt > 0)
                    len += cnt;
            }
        }
        ctx_lens[t] = (int32_t)len;
    }
    return 0;
}

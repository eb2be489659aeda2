/*
 * CPU oracle for the AB-Sparse decode path.  TEST INFRASTRUCTURE ONLY: the
 * parity tests, the smoke check and the benchmark's CPU-baseline leg call
 * it; the library and its kernels never do, and it shares no code with them.
 *
 * Source: "AB-Sparse: Sparse Attention with Adaptive Block Size for Accurate
 * and Efficient Long-Context Inference" (arXiv 2605.12110), as shown on its
 * Pith review page.  Figure 1 names the four stages this file follows, in
 * order: a block representation (the centroid), dot-product estimation of an
 * importance score per block, top-K selection, and sparse attention over the
 * chosen blocks.  Figure 8's mapping residue fixes that 16-token physical
 * pages are grouped into per-head logical blocks (stride = pages per block)
 * and that heads with different strides select different numbers of blocks
 * for the same number of pages; Figure 8's caption fixes INT4 asymmetric
 * per-channel quantization of the centroids; Figure 5's text fixes that the
 * block size of a head is static.  Exact attention over the kept tokens is
 * the textbook softmax (FlashAttention, the page's reference list).
 *
 * Readings where the page is silent (each is stated at its function):
 * mean-key centroid over the valid tokens of a block; one (scale, lo) pair
 * per (sequence, KV head, channel) over all blocks of that head; float zero
 * point, fp32 scale and quotient, round-half-even; query of a GQA group =
 * sum of its heads' queries; K = min(N, max(1, budget / block_size));
 * ties to the lower block index; selections reported in ascending order;
 * softmax scale passed in, no mask.
 *
 * Arithmetic: fp64 everywhere, except the quantizer, whose fp32 steps are
 * the ones that decide an integer code and are done in fp32 on purpose.
 * Plain loops; OpenMP only splits independent (sequence, head) pairs.
 *
 * Layouts (shared by definition with the library, not by code):
 *   cache  [num_pages][Hkv][16][D]   element = fp32, or bf16 bit pattern
 *   page_table [B][max_pages] int32  token t of sequence b is at
 *                                    page_table[b][t/16], slot t%16
 *   q      [B][Hq][D]                query head i reads KV head i / (Hq/Hkv)
 *   blocks of (b, h) are numbered j = 0..N-1, N = ceil(L_b / bs_h), and
 *   stored b-major, then h, then j ("CSR" order).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PAGE 16

/* ---- element access ---------------------------------------------------- */

static double elem(const void *base, int is_bf16, size_t i)
{
    if (is_bf16) {
        uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)base)[i];
}

/* channel d of token t of sequence b, KV head h, read through the page table */
static double cache_at(const void *cache, int is_bf16, const int32_t *page_table,
                       int max_pages, int Hkv, int D, int b, int h, int64_t t, int d)
{
    int64_t page = page_table[(int64_t)b * max_pages + t / PAGE];
    size_t i = ((((size_t)page * Hkv + h) * PAGE + (size_t)(t % PAGE)) * D) + d;
    return elem(cache, is_bf16, i);
}

static int64_t n_blocks(int64_t L, int bs) { return (L + bs - 1) / bs; }

int64_t oracle_total_blocks(int B, int Hkv, const int32_t *seq_lens, const int32_t *block_size)
{
    int64_t n = 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hkv; ++h)
            n += n_blocks(seq_lens[b], block_size[h]);
    return n;
}

/* first block row of (b, h) in CSR order */
static int64_t first_block(int b, int h, int Hkv, const int32_t *seq_lens, const int32_t *block_size)
{
    int64_t n = 0;
    for (int bb = 0; bb < b; ++bb)
        for (int hh = 0; hh < Hkv; ++hh)
            n += n_blocks(seq_lens[bb], block_size[hh]);
    for (int hh = 0; hh < h; ++hh)
        n += n_blocks(seq_lens[b], block_size[hh]);
    return n;
}

/* K for (b, h): the token budget buys floor(budget / bs) blocks, at least
 * one, never more than exist (equal pages per head, Figure 8 residue). */
static int64_t k_for(int64_t N, int bs, int budget)
{
    int64_t k = budget / bs;
    if (k < 1) k = 1;
    if (k > N) k = N;
    return k;
}

int64_t oracle_k(int64_t L, int bs, int budget) { return k_for(n_blocks(L, bs), bs, budget); }

/* ---- stage 1: block representation -------------------------------------- */

/* Centroid of block j = arithmetic mean of the keys of its valid tokens
 * [j*bs, min((j+1)*bs, L)), summed in fp64 and rounded once to fp32.
 * block_size may be any value >= 1 here (1 gives centroid = key). */
void oracle_centroids(int B, int Hkv, int D, int max_pages, int is_bf16,
                      const void *k_cache, const int32_t *page_table,
                      const int32_t *seq_lens, const int32_t *block_size,
                      float *centroids /* [total_blocks][D] */)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t L = seq_lens[b];
            int bs = block_size[h];
            int64_t N = n_blocks(L, bs);
            int64_t row0 = first_block(b, h, Hkv, seq_lens, block_size);
            double *acc = (double *)malloc(sizeof(double) * D);
            for (int64_t j = 0; j < N; ++j) {
                int64_t t0 = j * bs;
                int64_t t1 = t0 + bs < L ? t0 + bs : L;
                for (int d = 0; d < D; ++d) acc[d] = 0.0;
                for (int64_t t = t0; t < t1; ++t)
                    for (int d = 0; d < D; ++d)
                        acc[d] += cache_at(k_cache, is_bf16, page_table, max_pages, Hkv, D, b, h, t, d);
                for (int d = 0; d < D; ++d)
                    centroids[(row0 + j) * D + d] = (float)(acc[d] / (double)(t1 - t0));
            }
            free(acc);
        }
    }
}

/* ---- stage 1b: INT4 asymmetric per-channel quantization ----------------- */

/* Per (b, h, d): lo = min_j c_j[d], hi = max_j c_j[d] over the head's blocks;
 * scale = (hi - lo) / 15 and code = clamp(rint((c - lo) / scale), 0, 15),
 * each of those fp32 operations rounded to fp32 (the integer code is decided
 * in fp32); a constant channel (scale 0) gets code 0 and dequantizes to lo.
 * codes are one byte per channel here (values 0..15), [total_blocks][D]. */
void oracle_quantize(int B, int Hkv, int D, const int32_t *seq_lens, const int32_t *block_size,
                     const float *centroids, uint8_t *codes, float *scale, float *lo)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t N = n_blocks(seq_lens[b], block_size[h]);
            int64_t row0 = first_block(b, h, Hkv, seq_lens, block_size);
            for (int d = 0; d < D; ++d) {
                float mn = centroids[row0 * D + d], mx = mn;
                for (int64_t j = 1; j < N; ++j) {
                    float c = centroids[(row0 + j) * D + d];
                    if (c < mn) mn = c;
                    if (c > mx) mx = c;
                }
                volatile float range = mx - mn;          /* fp32 subtraction */
                volatile float s = range / 15.0f;        /* fp32 division */
                scale[((size_t)b * Hkv + h) * D + d] = s;
                lo[((size_t)b * Hkv + h) * D + d] = mn;
                for (int64_t j = 0; j < N; ++j) {
                    uint8_t code = 0;
                    if (s > 0.0f) {
                        volatile float diff = centroids[(row0 + j) * D + d] - mn;
                        volatile float quot = diff / s;
                        float r = rintf(quot);
                        if (r < 0.0f) r = 0.0f;
                        if (r > 15.0f) r = 15.0f;
                        code = (uint8_t)r;
                    }
                    codes[(row0 + j) * D + d] = code;
                }
            }
        }
    }
}

/* ---- stage 1c: centroids kept current while decoding -------------------- */

/* The page fixes a static block size per head (Figure 5's text) and INT4
 * per-channel centroids (Figure 8) but not how they follow appended tokens.
 * Reading: after sequence b grew from prev_b to L_b tokens (1 <= prev_b <=
 * L_b), every block holding one of the tokens [prev_b - 1, L_b) -- blocks
 * j = (prev_b - 1) / bs .. N - 1, so the last, possibly partial block is
 * always redone -- gets its centroid recomputed exactly as in
 * oracle_centroids and coded in format fmt (see oracle_quantize_fmt) with the
 * head's stored (scale, lo), the code clamped to the format's range.
 * out_of_range[b][h] counts the (block, channel) codes that were clamped: the
 * rounded quotient fell outside the range (0..15, 0..255, or -7..7 for the
 * symmetric form), or, in a constant channel (scale 0), the centroid differs
 * from what code 0 stands for (lo; 0 for the symmetric form); for bf16, a
 * finite centroid that rounds to an infinity.  A caller rebuilds the whole
 * layer when it wants a new range.  Block j of (b, h) is row
 * row_off[b*Hkv + h] + j of codes (one value per channel), so the offsets may
 * leave room for blocks still to come. */
void oracle_update(int fmt, int B, int Hkv, int D, int max_pages, int is_bf16,
                   const void *k_cache, const int32_t *page_table,
                   const int32_t *seq_lens, const int32_t *prev_lens, const int32_t *block_size,
                   const int64_t *row_off, const float *scale, const float *lo,
                   uint16_t *codes /* [rows][D] */, int32_t *out_of_range /* [B][Hkv] */)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t L = seq_lens[b];
            int bs = block_size[h];
            int64_t N = n_blocks(L, bs);
            int64_t j_first = (prev_lens[b] - 1) / bs;
            int64_t row0 = row_off[(int64_t)b * Hkv + h];
            const float *sc = scale + ((size_t)b * Hkv + h) * D;
            const float *zp = lo + ((size_t)b * Hkv + h) * D;
            double *acc = (double *)malloc(sizeof(double) * D);
            int32_t clamped = 0;
            for (int64_t j = j_first; j < N; ++j) {
                int64_t t0 = j * bs;
                int64_t t1 = t0 + bs < L ? t0 + bs : L;
                for (int d = 0; d < D; ++d) acc[d] = 0.0;
                for (int64_t t = t0; t < t1; ++t)
                    for (int d = 0; d < D; ++d)
                        acc[d] += cache_at(k_cache, is_bf16, page_table, max_pages, Hkv, D, b, h, t, d);
                for (int d = 0; d < D; ++d) {
                    float c = (float)(acc[d] / (double)(t1 - t0));
                    uint16_t code = 0;
                    if (fmt == 4) {
                        uint32_t u;
                        memcpy(&u, &c, 4);
                        code = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                        uint32_t back = (uint32_t)code << 16;
                        float f;
                        memcpy(&f, &back, 4);
                        if (isinf(f) && !isinf(c)) ++clamped;
                    } else if (fmt == 1) {
                        float r = 0.0f;
                        if (sc[d] > 0.0f) {
                            volatile float quot = c / sc[d];
                            r = rintf(quot);
                            if (r < -7.0f || r > 7.0f) ++clamped;
                            if (r < -7.0f) r = -7.0f;
                            if (r > 7.0f) r = 7.0f;
                        } else if (c != 0.0f) {
                            ++clamped;
                        }
                        code = (uint16_t)(r + 8.0f);
                    } else {
                        float top = fmt == 2 ? 255.0f : 15.0f;
                        if (sc[d] > 0.0f) {
                            volatile float diff = c - zp[d];
                            volatile float quot = diff / sc[d];
                            float r = rintf(quot);
                            if (r < 0.0f || r > top) ++clamped;
                            if (r < 0.0f) r = 0.0f;
                            if (r > top) r = top;
                            code = (uint16_t)r;
                        } else if (c != zp[d]) {
                            ++clamped;
                        }
                    }
                    codes[(row0 + j) * D + d] = code;
                }
            }
            out_of_range[(int64_t)b * Hkv + h] = clamped;
            free(acc);
        }
    }
}

/* ---- stage 1d: other centroid formats (precision variants) -------------- */

/* Figure 8 compares centroid precisions; the library can store the centroids
 * in five formats.  Per (b, h) over its blocks j and channels d:
 *   0  INT4 asymmetric per channel (oracle_quantize): lo = min_j c, scale =
 *      (max_j c - lo) / 15, code = clamp(rint((c - lo) / scale), 0, 15);
 *   1  INT4 symmetric per channel: a = max_j |c|, scale = a / 7,
 *      q = clamp(rint(c / scale), -7, 7), stored as q + 8; dequantized q*scale
 *      (lo is reported as -8*scale, the same value in the asymmetric form);
 *   2  INT8 asymmetric per channel: as 0 with 255 levels, code 0..255;
 *   3  INT4 asymmetric per (sequence, head): one lo = min over j and d, one
 *      scale = (max - lo) / 15 for every channel (reported per channel);
 *   4  bf16: the fp32 centroid rounded to bf16 (nearest, ties to even).
 * Each fp32 step that decides an integer code is an fp32 operation; a zero
 * scale gives code 0 (format 1: q = 0).  codes: [total_blocks][D] values
 * (format 4: bf16 bit patterns); deq: the dequantized centroids in fp64. */
void oracle_quantize_fmt(int fmt, int B, int Hkv, int D, const int32_t *seq_lens, const int32_t *block_size,
                         const float *centroids, uint16_t *codes, float *scale, float *lo, double *deq)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t N = n_blocks(seq_lens[b], block_size[h]);
            int64_t row0 = first_block(b, h, Hkv, seq_lens, block_size);
            float *sc = scale + ((size_t)b * Hkv + h) * D;
            float *zp = lo + ((size_t)b * Hkv + h) * D;
            float tmn = centroids[row0 * D], tmx = tmn;          /* format 3: over the whole head */
            for (int64_t j = 0; j < N; ++j)
                for (int d = 0; d < D; ++d) {
                    float c = centroids[(row0 + j) * D + d];
                    if (c < tmn) tmn = c;
                    if (c > tmx) tmx = c;
                }
            for (int d = 0; d < D; ++d) {
                float mn = centroids[row0 * D + d], mx = mn;
                for (int64_t j = 1; j < N; ++j) {
                    float c = centroids[(row0 + j) * D + d];
                    if (c < mn) mn = c;
                    if (c > mx) mx = c;
                }
                if (fmt == 3) {
                    mn = tmn;
                    mx = tmx;
                }
                volatile float s = 0.0f;
                float z = 0.0f;
                if (fmt == 1) {
                    float a = -mn > mx ? -mn : mx;              /* max |c| */
                    s = a / 7.0f;
                    z = -8.0f * s;
                } else if (fmt != 4) {
                    volatile float range = mx - mn;
                    s = range / (fmt == 2 ? 255.0f : 15.0f);
                    z = mn;
                }
                sc[d] = fmt == 4 ? 0.0f : s;
                zp[d] = fmt == 4 ? 0.0f : z;
                for (int64_t j = 0; j < N; ++j) {
                    float c = centroids[(row0 + j) * D + d];
                    size_t i = (size_t)(row0 + j) * D + d;
                    if (fmt == 4) {
                        uint32_t u;
                        memcpy(&u, &c, 4);
                        uint16_t hb = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
                        uint32_t back = (uint32_t)hb << 16;
                        float f;
                        memcpy(&f, &back, 4);
                        codes[i] = hb;
                        deq[i] = (double)f;
                    } else if (fmt == 1) {
                        float r = 0.0f;
                        if (s > 0.0f) {
                            volatile float quot = c / s;
                            r = rintf(quot);
                            if (r < -7.0f) r = -7.0f;
                            if (r > 7.0f) r = 7.0f;
                        }
                        codes[i] = (uint16_t)(r + 8.0f);
                        deq[i] = (double)r * (double)s;
                    } else {
                        float top = fmt == 2 ? 255.0f : 15.0f, r = 0.0f;
                        if (s > 0.0f) {
                            volatile float diff = c - mn;
                            volatile float quot = diff / s;
                            r = rintf(quot);
                            if (r < 0.0f) r = 0.0f;
                            if (r > top) r = top;
                        }
                        codes[i] = (uint16_t)r;
                        deq[i] = (double)r * (double)s + (double)mn;
                    }
                }
            }
        }
    }
}

/* ---- stage 2: dot-product estimation ------------------------------------ */

/* Importance score of block j of (b, h): the group query qbar = sum of the
 * G query heads that share KV head h, dotted with the dequantized centroid
 * code*scale + lo, all in fp64.  No softmax scale: it does not change the
 * order.  scores: [total_blocks] in CSR order. */
void oracle_scores(int B, int Hq, int Hkv, int D, int is_bf16, const void *q,
                   const int32_t *seq_lens, const int32_t *block_size,
                   const uint8_t *codes, const float *scale, const float *lo, double *scores)
{
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t N = n_blocks(seq_lens[b], block_size[h]);
            int64_t row0 = first_block(b, h, Hkv, seq_lens, block_size);
            double *qbar = (double *)calloc((size_t)D, sizeof(double));
            for (int g = 0; g < G; ++g)
                for (int d = 0; d < D; ++d)
                    qbar[d] += elem(q, is_bf16, ((size_t)b * Hq + (size_t)h * G + g) * D + d);
            const float *sc = scale + ((size_t)b * Hkv + h) * D;
            const float *zp = lo + ((size_t)b * Hkv + h) * D;
            for (int64_t j = 0; j < N; ++j) {
                double s = 0.0;
                for (int d = 0; d < D; ++d) {
                    double chat = (double)codes[(row0 + j) * D + d] * (double)sc[d] + (double)zp[d];
                    s += qbar[d] * chat;
                }
                scores[row0 + j] = s;
            }
            free(qbar);
        }
    }
}

/* The same estimation from dequantized centroids of any format:
 * score_j = qbar . chat_j in fp64; chat: [total_blocks][D]. */
void oracle_scores_dense(int B, int Hq, int Hkv, int D, int is_bf16, const void *q,
                         const int32_t *seq_lens, const int32_t *block_size, const double *chat, double *scores)
{
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t N = n_blocks(seq_lens[b], block_size[h]);
            int64_t row0 = first_block(b, h, Hkv, seq_lens, block_size);
            double *qbar = (double *)calloc((size_t)D, sizeof(double));
            for (int g = 0; g < G; ++g)
                for (int d = 0; d < D; ++d)
                    qbar[d] += elem(q, is_bf16, ((size_t)b * Hq + (size_t)h * G + g) * D + d);
            for (int64_t j = 0; j < N; ++j) {
                double s = 0.0;
                for (int d = 0; d < D; ++d) s += qbar[d] * chat[(row0 + j) * D + d];
                scores[row0 + j] = s;
            }
            free(qbar);
        }
    }
}

/* ---- stage 3: top-K selection ------------------------------------------- */

typedef struct { double s; int64_t j; } ranked;

/* higher score first; equal scores: lower block index first */
static int by_rank(const void *a, const void *b)
{
    const ranked *x = (const ranked *)a, *y = (const ranked *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int by_index(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Keep the K best blocks of each (b, h), ranked by (score desc, index asc);
 * write them in ascending block order to sel[b][h][0..K-1] (row stride
 * sel_cap) and K to count[b][h].  Unused sel slots are left untouched. */
void oracle_select(int B, int Hkv, const int32_t *seq_lens, const int32_t *block_size,
                   int budget, const double *scores, int32_t *sel, int sel_cap, int32_t *count)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t N = n_blocks(seq_lens[b], block_size[h]);
            int64_t K = k_for(N, block_size[h], budget);
            int64_t row0 = first_block(b, h, Hkv, seq_lens, block_size);
            ranked *r = (ranked *)malloc(sizeof(ranked) * (size_t)N);
            for (int64_t j = 0; j < N; ++j) { r[j].s = scores[row0 + j]; r[j].j = j; }
            qsort(r, (size_t)N, sizeof(ranked), by_rank);
            int32_t *out = sel + ((size_t)b * Hkv + h) * sel_cap;
            int64_t k = K < sel_cap ? K : sel_cap;
            for (int64_t i = 0; i < k; ++i) out[i] = (int32_t)r[i].j;
            qsort(out, (size_t)k, sizeof(int32_t), by_index);
            count[(size_t)b * Hkv + h] = (int32_t)k;
            free(r);
        }
    }
}

/* ---- stage 4: sparse attention ------------------------------------------ */

/* For each query head i of KV head h: the kept tokens T are the union of the
 * selected blocks' token ranges (clipped to L_b).  z_t = sm_scale * q_i.k_t,
 * out_i = sum_t softmax(z)_t v_t, lse_i = ln sum_t exp(z_t); fp64 with the
 * maximum subtracted.  out: [B][Hq][D], lse: [B][Hq]. */
void oracle_attend(int B, int Hq, int Hkv, int D, int max_pages, int is_bf16,
                   const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *page_table, const int32_t *seq_lens, const int32_t *block_size,
                   const int32_t *sel, int sel_cap, const int32_t *count, double sm_scale,
                   double *out, double *lse)
{
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t L = seq_lens[b];
            int bs = block_size[h];
            const int32_t *blk = sel + ((size_t)b * Hkv + h) * sel_cap;
            int64_t K = count[(size_t)b * Hkv + h];
            int64_t ntok = 0;
            int64_t *tok = (int64_t *)malloc(sizeof(int64_t) * (size_t)(K * bs + 1));
            for (int64_t i = 0; i < K; ++i)
                for (int64_t t = (int64_t)blk[i] * bs; t < (int64_t)(blk[i] + 1) * bs && t < L; ++t)
                    tok[ntok++] = t;
            double *z = (double *)malloc(sizeof(double) * (size_t)(ntok + 1));
            for (int g = 0; g < G; ++g) {
                int i = h * G + g;
                size_t qrow = ((size_t)b * Hq + i) * D;
                double m = -INFINITY;
                for (int64_t n = 0; n < ntok; ++n) {
                    double s = 0.0;
                    for (int d = 0; d < D; ++d)
                        s += elem(q, is_bf16, qrow + d) *
                             cache_at(k_cache, is_bf16, page_table, max_pages, Hkv, D, b, h, tok[n], d);
                    z[n] = sm_scale * s;
                    if (z[n] > m) m = z[n];
                }
                double denom = 0.0;
                for (int64_t n = 0; n < ntok; ++n) {
                    z[n] = exp(z[n] - m);                 /* unnormalized weight */
                    denom += z[n];
                }
                for (int d = 0; d < D; ++d) {
                    double acc = 0.0;
                    for (int64_t n = 0; n < ntok; ++n)
                        acc += z[n] * cache_at(v_cache, is_bf16, page_table, max_pages, Hkv, D, b, h, tok[n], d);
                    out[qrow + d] = ntok > 0 ? acc / denom : 0.0;
                }
                lse[(size_t)b * Hq + i] = ntok > 0 ? m + log(denom) : -INFINITY;
            }
            free(z);
            free(tok);
        }
    }
}

/* ---- calibration: attention mass kept by a selection -------------------- */

/* Figure 3 of the page plots, per head, recall against block size,
 * normalized by the recall at block size 16.  Reading: the recall of a
 * selection for query head i is the share of i's exact attention over all
 * L_b tokens that falls on the kept tokens,
 *     mass_i = sum_{t kept} exp(z_t) / sum_{t < L_b} exp(z_t),
 * z_t = sm_scale * q_i . k_t, in fp64 (both sums taken with the maximum
 * over all tokens subtracted).  mass: [B][Hq]. */
void oracle_attention_mass(int B, int Hq, int Hkv, int D, int max_pages, int is_bf16,
                           const void *q, const void *k_cache, const int32_t *page_table,
                           const int32_t *seq_lens, const int32_t *block_size,
                           const int32_t *sel, int sel_cap, const int32_t *count, double sm_scale,
                           double *mass)
{
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hkv; ++h) {
            int64_t L = seq_lens[b];
            int bs = block_size[h];
            const int32_t *blk = sel + ((size_t)b * Hkv + h) * sel_cap;
            int64_t K = count[(size_t)b * Hkv + h];
            unsigned char *kept = (unsigned char *)calloc((size_t)L, 1);
            for (int64_t i = 0; i < K; ++i)
                for (int64_t t = (int64_t)blk[i] * bs; t < (int64_t)(blk[i] + 1) * bs && t < L; ++t)
                    kept[t] = 1;
            double *z = (double *)malloc(sizeof(double) * (size_t)L);
            for (int g = 0; g < G; ++g) {
                int i = h * G + g;
                size_t qrow = ((size_t)b * Hq + i) * D;
                double m = -INFINITY;
                for (int64_t t = 0; t < L; ++t) {
                    double s = 0.0;
                    for (int d = 0; d < D; ++d)
                        s += elem(q, is_bf16, qrow + d) *
                             cache_at(k_cache, is_bf16, page_table, max_pages, Hkv, D, b, h, t, d);
                    z[t] = sm_scale * s;
                    if (z[t] > m) m = z[t];
                }
                double all = 0.0, in = 0.0;
                for (int64_t t = 0; t < L; ++t) {
                    double e = exp(z[t] - m);
                    all += e;
                    if (kept[t]) in += e;
                }
                mass[(size_t)b * Hq + i] = in / all;
            }
            free(z);
            free(kept);
        }
    }
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

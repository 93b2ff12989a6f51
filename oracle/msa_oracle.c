/*
 * msa_oracle.c -- plain, slow, obviously-correct CPU oracle for the hot path
 * of MiniMax Sparse Attention (MSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  It shares no
 * code, header, table or helper with the GPU library (libmsa): it includes
 * nothing from it and the GPU library includes nothing from here.
 *
 * Every routine follows the definition of the step directly: loops in the
 * order the definition reads, no tiling, no fusion, no reordering.  bf16
 * inputs are widened exactly (a bf16 is the top 16 bits of an IEEE float) and
 * every sum is accumulated in double precision.
 *
 * Sources (the pages describing the method):
 *  [T]  "Together AI 解析如何高效服务 MiniMax M3：1M token 上下文与多模态推理优化"
 *       (aihot.news), sections 架构/特性 (architecture), KV 块主序稀疏注意力
 *       (KV-block-major sparse attention), 将 MSA 与分页注意力集成 (paged
 *       attention integration), 解码索引评分内核优化 (decode index-scoring
 *       kernel).
 *  [J]  "MiniMax-M3の効率的な推論サービス" (news.chathome.org), the paragraphs on
 *       MSA, the block-major kernel, paged integration and index scoring.
 *  [N]  "NVIDIA 加速インフラ上で MiniMax M3 を活用した長文脈推論..." (news.ainew.jp),
 *       the paragraph on MiniMax Sparse Attention.
 *
 * Readings taken where the pages leave a step open (each one is also listed in
 * the design notes):
 *  - block score = max over the block's causally visible tokens of
 *    sum_j (q_j . k_t) / sqrt(d_idx); the pages say only that each 128-token
 *    block is reduced to one score.
 *  - the own (causal) block is always selected, on top of the k ranked
 *    candidates; candidates are the scored blocks strictly before it.
 *  - ranking is score descending, ties to the lower block index; the selected
 *    list is written in ascending block order and padded with -1.
 *  - softmax scale is a parameter; log-sum-exp uses the natural logarithm.
 *
 * Parity pins: every function here is pinned by tests that do not re-type its
 * formula (closed forms, exact integer brute force through a library matmul,
 * a set-property brute force for top-k, dense causal attention through a
 * library attention routine, merge identities).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BLK 128 /* tokens per KV block = tokens per cache page ([T] decode index scoring) */

/* Exact widening of a bf16 bit pattern. */
static double bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int orc_block_tokens(void) { return ORC_BLK; }

/*
 * Index score ([T] 解码索引评分内核优化: query-side index vectors are compared
 * with the candidate key-side index vectors and every 128-token KV block is
 * reduced to a single score; the range of candidate blocks and the mask are
 * per request and KV group).
 *
 * For row r (request req, position pos, own block own = pos / 128), group g and
 * block b in [0, nb):
 *   - b == own, or lo <= b < own     : scored
 *   - otherwise                      : -inf
 * A scored block's value is max over tokens t of b with b*128 + t <= pos of
 *   ( sum_{j < n_idx} sum_{d < d_idx} q_idx[r][g][j][d] * k_idx[page][g][t][d] ) / sqrt(d_idx)
 * where page = block_table[req][b].
 *
 * q_idx    : bf16 bits, [rows][G][n_idx][d_idx], contiguous
 * k_idx    : bf16 bits, element (page, g, t, d) at page*ps + g*gs + t*ts + d
 * blk_lo   : [num_reqs][G] or NULL (NULL means lo = 0)
 * row_req  : [rows] or NULL (NULL means row r belongs to request r)
 * scores   : [rows][G][nb]
 */
void orc_index_score(int32_t rows, int32_t G, int32_t n_idx, int32_t d_idx,
                     const uint16_t *q_idx,
                     const uint16_t *k_idx, int64_t ps, int64_t gs, int64_t ts,
                     const int32_t *block_table, int32_t bt_stride,
                     const int32_t *row_req, const int32_t *row_pos,
                     const int32_t *blk_lo, int32_t nb, double *scores)
{
    const double inv_sqrt_d = 1.0 / sqrt((double)d_idx);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int32_t r = 0; r < rows; ++r) {
        for (int32_t g = 0; g < G; ++g) {
            const int32_t req = row_req ? row_req[r] : r;
            const int32_t pos = row_pos[r];
            const int32_t own = pos / ORC_BLK;
            const int32_t lo = blk_lo ? blk_lo[(int64_t)req * G + g] : 0;
            const uint16_t *q = q_idx + ((int64_t)r * G + g) * n_idx * d_idx;
            double *out = scores + ((int64_t)r * G + g) * nb;
            for (int32_t b = 0; b < nb; ++b) {
                const int scored = (b == own) || (b >= lo && b < own);
                if (!scored) {
                    out[b] = -INFINITY;
                    continue;
                }
                const int64_t page = block_table[(int64_t)req * bt_stride + b];
                double best = -INFINITY;
                for (int32_t t = 0; t < ORC_BLK; ++t) {
                    if ((int64_t)b * ORC_BLK + t > pos)
                        break; /* causal mask inside the own block */
                    const uint16_t *k = k_idx + page * ps + (int64_t)g * gs + (int64_t)t * ts;
                    double sum = 0.0;
                    for (int32_t j = 0; j < n_idx; ++j) {
                        double dot = 0.0;
                        for (int32_t d = 0; d < d_idx; ++d)
                            dot += bf16_to_f64(q[j * d_idx + d]) * bf16_to_f64(k[d]);
                        sum += dot;
                    }
                    const double s = sum * inv_sqrt_d;
                    if (s > best)
                        best = s;
                }
                out[b] = best;
            }
        }
    }
}

/* Ranking order of the top-k: score descending, then block index ascending. */
typedef struct {
    float score;
    int32_t block;
} orc_cand_t;

static int cand_rank_cmp(const void *pa, const void *pb)
{
    const orc_cand_t *a = (const orc_cand_t *)pa, *b = (const orc_cand_t *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->block < b->block) ? -1 : (a->block > b->block);
}

static int int_asc_cmp(const void *pa, const void *pb)
{
    const int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/*
 * Top-k block selection ([T] 架构/特性: the score part picks the K most relevant
 * blocks for each KV group; [T] 解码索引评分内核优化: top-k boundary per request
 * and group).
 *
 * For row r and group g, with own = row_pos[r] / 128:
 *   candidates C = { b < own : scores[r][g][b] != -inf }
 *   rank C by (score descending, block ascending), keep the first min(k, |C|),
 *   add own, write in ascending block order into sel[r][g][0 .. k], pad with -1.
 * The decision is taken on the fp32 scores the caller passes.
 *
 * scores : [rows][G][score_stride] fp32 (score_stride > own for every row)
 * sel    : [rows][G][k + 1]
 */
void orc_topk(int32_t rows, int32_t G, const float *scores, int32_t score_stride,
              const int32_t *row_pos, int32_t k, int32_t *sel)
{
    const int32_t nslot = k + 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int32_t r = 0; r < rows; ++r) {
        for (int32_t g = 0; g < G; ++g) {
            const int32_t own = row_pos[r] / ORC_BLK;
            const float *s = scores + ((int64_t)r * G + g) * score_stride;
            orc_cand_t *cand = (orc_cand_t *)malloc(sizeof(orc_cand_t) * (size_t)(own > 0 ? own : 1));
            int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * (size_t)nslot);
            int32_t n = 0;
            for (int32_t b = 0; b < own; ++b) {
                if (s[b] != -INFINITY) {
                    cand[n].score = s[b];
                    cand[n].block = b;
                    ++n;
                }
            }
            qsort(cand, (size_t)n, sizeof(orc_cand_t), cand_rank_cmp);
            const int32_t keep = (k < n) ? k : n;
            for (int32_t i = 0; i < keep; ++i)
                chosen[i] = cand[i].block;
            chosen[keep] = own;
            qsort(chosen, (size_t)(keep + 1), sizeof(int32_t), int_asc_cmp);
            int32_t *out = sel + ((int64_t)r * G + g) * nslot;
            for (int32_t i = 0; i < nslot; ++i)
                out[i] = (i <= keep) ? chosen[i] : -1;
            free(cand);
            free(chosen);
        }
    }
}

/*
 * Page table over the selected blocks ([T] 将 MSA 与分页注意力集成: build a page
 * table from the selected blocks, one row per (query row, KV group)).
 *   pt[r][g][s] = block_table[req][sel[r][g][s]],   -1 stays -1.
 */
void orc_page_table(int32_t rows, int32_t G, int32_t nslot, const int32_t *sel,
                    const int32_t *row_req, const int32_t *block_table, int32_t bt_stride,
                    int32_t *pt)
{
    for (int32_t r = 0; r < rows; ++r) {
        const int32_t req = row_req ? row_req[r] : r;
        for (int32_t g = 0; g < G; ++g) {
            for (int32_t s = 0; s < nslot; ++s) {
                const int64_t i = ((int64_t)r * G + g) * nslot + s;
                pt[i] = (sel[i] < 0) ? -1 : block_table[(int64_t)req * bt_stride + sel[i]];
            }
        }
    }
}

/* Softmax attention of one query head over a list of (page, block) pairs,
 * visiting the causally visible tokens of each block in ascending position.
 * Writes o[D] and returns lse = m + ln(sum exp(z - m)); with no token at all
 * it writes zeros and returns -inf. */
static double attend(int32_t D, const uint16_t *q,
                     const uint16_t *kc, int64_t kps, int64_t kgs, int64_t kts,
                     const uint16_t *vc, int64_t vps, int64_t vgs, int64_t vts,
                     int32_t g, const int32_t *blocks, const int32_t *pages, int32_t n,
                     int32_t pos, double sm_scale, double *o)
{
    double m = -INFINITY;
    for (int32_t i = 0; i < n; ++i) {
        for (int32_t t = 0; t < ORC_BLK && (int64_t)blocks[i] * ORC_BLK + t <= pos; ++t) {
            const uint16_t *kr = kc + (int64_t)pages[i] * kps + (int64_t)g * kgs + (int64_t)t * kts;
            double z = 0.0;
            for (int32_t d = 0; d < D; ++d)
                z += bf16_to_f64(q[d]) * bf16_to_f64(kr[d]);
            z *= sm_scale;
            if (z > m) m = z;
        }
    }
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    if (m == -INFINITY)
        return -INFINITY;
    double l = 0.0;
    for (int32_t i = 0; i < n; ++i) {
        for (int32_t t = 0; t < ORC_BLK && (int64_t)blocks[i] * ORC_BLK + t <= pos; ++t) {
            const uint16_t *kr = kc + (int64_t)pages[i] * kps + (int64_t)g * kgs + (int64_t)t * kts;
            const uint16_t *vr = vc + (int64_t)pages[i] * vps + (int64_t)g * vgs + (int64_t)t * vts;
            double z = 0.0;
            for (int32_t d = 0; d < D; ++d)
                z += bf16_to_f64(q[d]) * bf16_to_f64(kr[d]);
            z *= sm_scale;
            const double p = exp(z - m);
            l += p;
            for (int32_t d = 0; d < D; ++d)
                o[d] += p * bf16_to_f64(vr[d]);
        }
    }
    for (int32_t d = 0; d < D; ++d) o[d] /= l;
    return m + log(l);
}

/*
 * Sparse attention, direct form ([T] 架构/特性: dense attention of the query
 * tokens over the selected blocks; the heads of one KV group share its
 * selection).  For row r and head h (group g = h / Hg): one softmax over the
 * union of the causally visible tokens of every selected block (sel >= 0).
 *
 * q          : bf16 bits [rows][G*Hg][D]
 * K, V       : bf16 bits, element (page, g, t, d) at page*ps + g*gs + t*ts + d
 * sel, pt    : [rows][G][nslot]  (block index and physical page; -1 = empty)
 * o          : [rows][G*Hg][D],  lse : [rows][G*Hg]
 */
void orc_attn(int32_t rows, int32_t G, int32_t Hg, int32_t D, const uint16_t *q,
              const uint16_t *kc, int64_t kps, int64_t kgs, int64_t kts,
              const uint16_t *vc, int64_t vps, int64_t vgs, int64_t vts,
              const int32_t *sel, const int32_t *pt, int32_t nslot,
              const int32_t *row_pos, double sm_scale, double *o, double *lse)
{
    const int32_t H = G * Hg;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int32_t r = 0; r < rows; ++r) {
        for (int32_t h = 0; h < H; ++h) {
            const int32_t g = h / Hg;
            int32_t *blocks = (int32_t *)malloc(sizeof(int32_t) * (size_t)nslot);
            int32_t *pages = (int32_t *)malloc(sizeof(int32_t) * (size_t)nslot);
            int32_t n = 0;
            for (int32_t s = 0; s < nslot; ++s) {
                const int64_t i = ((int64_t)r * G + g) * nslot + s;
                if (sel[i] >= 0) {
                    blocks[n] = sel[i];
                    pages[n] = pt[i];
                    ++n;
                }
            }
            lse[(int64_t)r * H + h] =
                attend(D, q + ((int64_t)r * H + h) * D, kc, kps, kgs, kts, vc, vps, vgs, vts,
                       g, blocks, pages, n, row_pos[r], sm_scale, o + ((int64_t)r * H + h) * D);
            free(blocks);
            free(pages);
        }
    }
}

/*
 * Per-block partial attention ([T] KV 块主序稀疏注意力: each KV block yields a
 * partial O that a final log-sum-exp reduction rescales and sums).  The same
 * softmax as orc_attn restricted to one selected block: slot s gives the
 * normalised partial o_part[r][h][s][:] and lse_part[r][h][s]; an empty slot
 * (sel = -1) gives o = 0 and lse = -inf.
 */
void orc_attn_partials(int32_t rows, int32_t G, int32_t Hg, int32_t D, const uint16_t *q,
                       const uint16_t *kc, int64_t kps, int64_t kgs, int64_t kts,
                       const uint16_t *vc, int64_t vps, int64_t vgs, int64_t vts,
                       const int32_t *sel, const int32_t *pt, int32_t nslot,
                       const int32_t *row_pos, double sm_scale, double *o_part, double *lse_part)
{
    const int32_t H = G * Hg;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int32_t r = 0; r < rows; ++r) {
        for (int32_t h = 0; h < H; ++h) {
            const int32_t g = h / Hg;
            for (int32_t s = 0; s < nslot; ++s) {
                const int64_t i = ((int64_t)r * G + g) * nslot + s;
                const int64_t out = ((int64_t)r * H + h) * nslot + s;
                const int32_t n = (sel[i] >= 0) ? 1 : 0;
                lse_part[out] = attend(D, q + ((int64_t)r * H + h) * D, kc, kps, kgs, kts,
                                       vc, vps, vgs, vts, g, &sel[i], &pt[i], n, row_pos[r],
                                       sm_scale, o_part + out * D);
            }
        }
    }
}

/*
 * Log-sum-exp merge of per-block partials ([T] KV 块主序稀疏注意力: the final
 * reduction rescales the partial O outputs by their log-sum-exp and sums them;
 * the formula itself did not survive on the page, this is the standard one).
 *   m = max_s lse_s  over slots with lse_s > -inf
 *   w_s = exp(lse_s - m),  o = sum_s w_s o_s / sum_s w_s,  lse = m + ln(sum_s w_s)
 * With no finite slot: o = 0 and lse = -inf.
 *
 * o_part : [rows][H][nslot][D],  lse_part : [rows][H][nslot]
 * o      : [rows][H][D],         lse      : [rows][H]
 */
void orc_lse_merge(int32_t rows, int32_t H, int32_t nslot, int32_t D,
                   const double *o_part, const double *lse_part, double *o, double *lse)
{
    for (int64_t rh = 0; rh < (int64_t)rows * H; ++rh) {
        const double *ls = lse_part + rh * nslot;
        double *out = o + rh * D;
        double m = -INFINITY;
        for (int32_t s = 0; s < nslot; ++s)
            if (ls[s] > m) m = ls[s];
        for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
        if (m == -INFINITY) {
            lse[rh] = -INFINITY;
            continue;
        }
        double wsum = 0.0;
        for (int32_t s = 0; s < nslot; ++s) {
            if (ls[s] == -INFINITY) continue;
            const double w = exp(ls[s] - m);
            wsum += w;
            for (int32_t d = 0; d < D; ++d)
                out[d] += w * o_part[(rh * nslot + s) * D + d];
        }
        for (int32_t d = 0; d < D; ++d) out[d] /= wsum;
        lse[rh] = m + log(wsum);
    }
}

/*
 * msa.h -- C ABI of libmsa, the MI355X (gfx950) hot path of MiniMax Sparse
 * Attention (MSA).
 *
 * The method (pages: "Together AI 解析如何高效服务 MiniMax M3" on aihot.news, section
 * 架构/特性; "MiniMax-M3の効率的な推論サービス" on news.chathome.org; the MSA
 * paragraph of "NVIDIA 加速インフラ上で MiniMax M3 を活用した長文脈推論..." on
 * news.ainew.jp) has two halves: a score part that picks, per KV group, the
 * most relevant 128-token KV blocks, and dense attention of the query heads
 * over only those blocks.  The six compute calls below are the steps of that
 * path: index scoring, top-k block selection, page-table build, sparse decode
 * attention, KV-block-major sparse prefill attention and the log-sum-exp merge.
 * Four more serve it: msa_topk_blocks_paged (selection and page table in one
 * launch), msa_sparse_attn_decode_select (selection, page table and decode
 * attention in one launch), msa_decode_step (the whole decode step, one
 * launch for short contexts and small batches) and msa_gather_pages (the
 * selected KV pages of a cache in host memory, loaded on demand into a device
 * pool).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every call returns an msa_status_t.  On an error nothing is launched and
 *    msa_last_error() holds a thread-local description.
 *  - Calls are asynchronous on the caller's HIP stream (NULL = the default
 *    stream).  They never synchronise and never allocate device memory.
 *  - The caller owns every buffer.  Array arguments are device pointers on the
 *    current device unless stated otherwise; the library keeps no pointer after
 *    a call returns.
 *  - Host-side validation covers scalars, pointers, alignment and strides.  The
 *    values inside device index arrays (row_pos, row_req, block_table, sel,
 *    page_table, blk_lo) cannot be checked from the host: keeping them in range
 *    is a precondition, and a violation is undefined behaviour (typically a
 *    memory fault reported by the caller's next synchronisation).
 *  - Outputs are written in full, padding included (-inf scores, -1 indices,
 *    zero partial outputs with -inf log-sum-exp).
 *  - bf16 is stored as its 16-bit pattern (the top half of an IEEE float).
 *  - Blocks and cache pages are 128 tokens (dims.blk must be 128).  Block b of
 *    a request covers positions [128 b, 128 b + 127]; a row at position pos
 *    owns block own = pos / 128 and sees positions <= pos only (causal).
 *  - The library is stateless and thread-safe.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MSA_OK = 0,
    MSA_ERR_NULL = 1,        /* a required pointer is NULL */
    MSA_ERR_INVALID = 2,     /* a size, stride or alignment is invalid */
    MSA_ERR_UNSUPPORTED = 3, /* valid but not implemented (e.g. D != 128) */
    MSA_ERR_WORKSPACE = 4,   /* workspace too small */
    MSA_ERR_HIP = 5          /* a HIP launch failed */
} msa_status_t;

/* A HIP stream (hipStream_t); NULL selects the default stream. */
typedef void *msa_stream_t;

/* Model dimensions.
 *   G      KV groups (KV heads)                       >= 1
 *   Hg     query heads per KV group; head h uses group h / Hg; Hg in {1,2,4,8,16}
 *   D      head dimension                             == 128
 *   n_idx  query-side index vectors per (row, group)  1 .. 16
 *   d_idx  index-vector dimension                     64 or 128
 *   blk    tokens per block and per cache page        == 128 */
typedef struct {
    int32_t G, Hg, D, n_idx, d_idx, blk;
} msa_dims_t;

/* A paged cache tensor: element (page, group, token, dim) of a bf16 cache lives
 * at base + page*page_stride + group*group_stride + token*token_stride + dim
 * (strides in elements; the dim stride is 1).  base must be 16-byte aligned
 * and every stride a multiple of 8.  The default layout [page][G][128][dim]
 * is page_stride = G*128*dim, group_stride = 128*dim, token_stride = dim; a
 * token-major cache [page][128][G][dim] is group_stride = dim,
 * token_stride = G*dim.
 *
 * The K and V caches of the attention calls may also live in pinned host
 * memory that is mapped into the device's address space (hipHostMalloc'd,
 * torch pin_memory): the kernels then read only the pages the selection names,
 * over the host link.  This is the pages' decoupled offload (未来工作 of the
 * aihot.news page): the full key index resident on the GPU, the KV cache in
 * CPU memory, loaded on demand from the top-k selection.  Results are
 * identical to a device-resident cache; the time is bound by the host link. */
typedef struct {
    const void *base;
    int64_t page_stride, group_stride, token_stride;
} msa_view_t;

/* ------------------------------------------------------------------ a1 / a6
 * msa_index_score -- block scores from the index vectors.
 * Pages: decode index-scoring section (解码索引评分内核优化) of the aihot.news
 * page: query-side index vectors are compared with every candidate key-side
 * index vector, each 128-token block reduces to a single score, and every
 * request and K group has its own candidate block range and mask.
 *
 * For row r (request req = row_req[r], position pos = row_pos[r], own = pos/128),
 * group g and block b in [0, score_stride):
 *     scored iff b == own or lo <= b < own   (lo = blk_lo[req][g], or 0)
 *     scores[r][g][b] = max over tokens t of block b with 128 b + t <= pos of
 *                       sum_{j < n_idx} dot(q_idx[r][g][j], k_idx[page][g][t]) / sqrt(d_idx)
 *     where page = block_table[req][b]; unscored blocks get -inf.
 * (The block reduction -- max over tokens of the summed index dot products --
 * is this library's reading; the pages leave it open.)
 *
 *   q_idx        bf16 [rows][G][n_idx][d_idx], contiguous, 16-byte aligned
 *   k_idx        key-index cache view, dim = d_idx
 *   block_table  int32 [num_reqs][bt_stride]: logical block -> physical page
 *   row_req      int32 [rows], or NULL when row r is request r
 *   row_pos      int32 [rows]
 *   blk_lo       int32 [num_reqs][G], or NULL for lo = 0
 *   num_reqs     number of requests (rows of block_table); a hint for the
 *                schedule (many rows per request -> tiled matrix-core path)
 *   scores       fp32 [rows][G][score_stride]; score_stride > own of every row
 * Accumulation is fp32 from bf16 inputs. */
msa_status_t msa_index_score(const msa_dims_t *dims, int32_t rows, const void *q_idx,
                             msa_view_t k_idx, const int32_t *block_table, int32_t bt_stride,
                             const int32_t *row_req, const int32_t *row_pos,
                             const int32_t *blk_lo, int32_t num_reqs, float *scores,
                             int32_t score_stride, msa_stream_t stream);

/* ------------------------------------------------------------------ a2 / a7
 * msa_topk_blocks -- per (row, group) block selection.
 * Pages: the score part picks the K most relevant blocks for each KV group
 * (架构/特性); each request and group has its own top-k boundary
 * (解码索引评分内核优化).
 *
 * Candidates are the blocks b < own with a score other than -inf.  They are
 * ranked by score descending, ties going to the lower block index; the first
 * min(k, #candidates) are kept, the own block is added, and the selection is
 * written in ascending block order to sel[r][g][0 .. k], padded with -1.
 *
 *   scores   fp32 [rows][G][score_stride] (as written by msa_index_score)
 *   row_pos  int32 [rows]
 *   k        0 <= k < 2^30; nslot = k + 1 entries per (row, group); the whole
 *            selection rows * G * (k + 1) must be below 2^31 - 1
 *            (MSA_ERR_INVALID otherwise, before anything is launched)
 *   sel      int32 [rows][G][k + 1] */
msa_status_t msa_topk_blocks(const msa_dims_t *dims, int32_t rows, const float *scores,
                             int32_t score_stride, const int32_t *row_pos, int32_t k,
                             int32_t *sel, msa_stream_t stream);

/* ------------------------------------------------------------------ a3
 * msa_build_page_table -- physical page of every selected block.
 * Pages: paged-attention integration section (将 MSA 与分页注意力集成): build a
 * page table from the selected blocks with the KV-group dimension folded into
 * the batch, so every (row, group) has a page list of its own.
 *
 *   page_table[r][g][s] = block_table[row_req[r]][sel[r][g][s]], -1 stays -1.
 *   sel, page_table  int32 [rows][G][nslot]
 *   row_req          int32 [rows] or NULL (row r is request r)
 *   block_table      int32 [num_reqs][bt_stride] */
msa_status_t msa_build_page_table(const msa_dims_t *dims, int32_t rows, const int32_t *sel,
                                  int32_t nslot, const int32_t *row_req,
                                  const int32_t *block_table, int32_t bt_stride,
                                  int32_t *page_table, msa_stream_t stream);

/* ------------------------------------------------------------------ a2 + a3
 * msa_topk_blocks_paged -- msa_topk_blocks and msa_build_page_table in one
 * kernel.  Pages: the new smaller kernels of the path (the top-k among them)
 * are named as fusion candidates (未来工作); the page table is the lookup of
 * 将 MSA 与分页注意力集成.
 *
 * Writes exactly what msa_topk_blocks (sel, nslot = k + 1) followed by
 * msa_build_page_table (page_table) write, bit for bit, with one launch and
 * without reading sel back.  Arguments as in those two calls. */
msa_status_t msa_topk_blocks_paged(const msa_dims_t *dims, int32_t rows, const float *scores,
                                   int32_t score_stride, const int32_t *row_pos, int32_t k,
                                   const int32_t *row_req, const int32_t *block_table,
                                   int32_t bt_stride, int32_t *sel, int32_t *page_table,
                                   msa_stream_t stream);

/* ------------------------------------------------------------------ a4
 * msa_sparse_attn_decode -- per-block partial attention for decode rows.
 * Pages: dense attention over the selected blocks (架构/特性), read through the
 * per-group page table (将 MSA 与分页注意力集成).
 *
 * For row r, head h (group g = h / Hg) and slot s with sel[r][g][s] = b >= 0:
 * softmax attention of q[r][h] over the tokens t of page page_table[r][g][s]
 * with 128 b + t <= row_pos[r], logits scaled by sm_scale:
 *     o_part[r][h][s][:] = normalised output (bf16),
 *     lse_part[r][s][h]  = m + ln(sum exp(z - m)) in natural log (fp32).
 * Empty slots get o = 0 and lse = -inf.  Combine with msa_lse_merge.
 *
 *   q         bf16 [rows][G*Hg][D], contiguous, 16-byte aligned
 *   k, v      key / value cache views, dim = D
 *   sel, page_table  int32 [rows][G][nslot]
 *   o_part    bf16 [rows][G*Hg][nslot][D];  lse_part fp32 [rows][nslot][G*Hg]
 *             (the LSEs of one (row, slot) are contiguous over the heads, so the
 *             Hg heads of a (row, group, slot) share one 32-byte sector)
 * bf16 inputs, fp32 accumulation on the matrix cores. */
msa_status_t msa_sparse_attn_decode(const msa_dims_t *dims, int32_t rows, const void *q,
                                    msa_view_t k, msa_view_t v, const int32_t *sel,
                                    const int32_t *page_table, int32_t nslot,
                                    const int32_t *row_pos, float sm_scale, void *o_part,
                                    float *lse_part, msa_stream_t stream);

/* ------------------------------------------------------------------ a2 + a3 + a4
 * msa_sparse_attn_decode_select -- msa_topk_blocks_paged and
 * msa_sparse_attn_decode in one launch.  Pages: the new smaller kernels of the
 * path, the top-k among them, are named as fusion candidates (未来工作); the
 * selection feeds the paged decode attention (将 MSA 与分页注意力集成).
 *
 * Writes exactly what msa_topk_blocks_paged (sel, page_table; nslot = k + 1)
 * followed by msa_sparse_attn_decode (o_part, lse_part) write, bit for bit.
 * With score_stride <= 1024 and rows * G * (k + 1) workgroups that the device
 * holds at once (one round; 1,280 on MI355X) it is one kernel: each workgroup
 * of a (row, group) repeats that group's top-k over its scores (integer
 * decisions, so every copy agrees) and attends to its own slot, so the decode
 * step loses one launch and the wait between the two kernels.  Otherwise
 * (longer score rows, or a batch whose later rounds would pay the repeated
 * top-k again) it runs the two kernels one after the other.  Arguments as in those two calls (sel and
 * page_table are outputs here; row_req may be NULL). */
msa_status_t msa_sparse_attn_decode_select(const msa_dims_t *dims, int32_t rows,
                                           const float *scores, int32_t score_stride, int32_t k,
                                           const int32_t *row_req, const int32_t *block_table,
                                           int32_t bt_stride, const void *q, msa_view_t kc,
                                           msa_view_t vc, const int32_t *row_pos, float sm_scale,
                                           int32_t *sel, int32_t *page_table, void *o_part,
                                           float *lse_part, msa_stream_t stream);

/* ------------------------------------------------------------------ f1
 * msa_decode_step -- the whole decode step: msa_index_score,
 * msa_topk_blocks_paged, msa_sparse_attn_decode and msa_lse_merge.  Pages: the
 * new smaller kernels of the path (the top-k among them) are named as fusion
 * candidates (未来工作 of the aihot.news page); the steps are those of the
 * decode index-scoring section (解码索引评分内核优化), the paged-attention
 * integration (将 MSA 与分页注意力集成) and the log-sum-exp reduction of the
 * per-block partials (KV 块主序稀疏注意力).
 *
 * Writes exactly what those calls write one after the other, bit for bit:
 * scores (fp32 [rows][G][score_stride]), sel and page_table (int32
 * [rows][G][k + 1]), o_part and lse_part (the slot partials), o (bf16
 * [rows][G*Hg][128]) and lse (fp32 [rows][G*Hg], may be NULL).  Arguments as
 * in those calls (nslot = k + 1; row_req and blk_lo may be NULL).  The one
 * exception: MSA_STEP_ONE_LAUNCH always scores with the streaming scan that
 * msa_index_score runs for decode batches; for batches of 64 or more rows per
 * request msa_index_score takes its row-tiled matrix-core scan instead, whose
 * scores agree with these to within rounding, not bit for bit.
 *
 *   sync  device int32 [MSA_DECODE_STEP_SYNC_WORDS(rows, G)], all zero before
 *         its first use; every call leaves it zero again (a call that hits
 *         the bound on its waits leaves word 2 set to 1: then the outputs are
 *         not valid).  Calls that share one sync array must not overlap.
 *         Used by MSA_STEP_ONE_LAUNCH only; may be NULL otherwise.
 *   mode
 *     MSA_STEP_ONE_LAUNCH  one kernel.  Its workgroups take tickets in the
 *                          order they start: the first ones run the scan, the
 *                          later ones one (row, group, slot) unit each, which
 *                          waits for its pair's scan (only ever for workgroups
 *                          that started before it, so every wait ends), then
 *                          selects and attends; the last unit of a pair
 *                          merges it.  Needs score_stride <= 1024
 *                          (MSA_ERR_UNSUPPORTED otherwise) and sync.  The scan's
 *                          waves each fence once per pair they finish.
 *     MSA_STEP_SEPARATE    the scan, then selection + attention
 *                          (msa_sparse_attn_decode_select), then the merge.
 *     MSA_STEP_AUTO        the faster form on MI355X: the separate launches at
 *                          every decode shape measured (issued back to back,
 *                          their launch gaps cost less than the single
 *                          launch's fences and waits: 21.2 against 25.1 us for
 *                          a 4K context, 196 against 415 us for 8 x 64K). 
 * Errors: as the four calls; MSA_ERR_INVALID for an unknown mode or rows * G
 * >= 2^28; MSA_ERR_NULL for MSA_STEP_ONE_LAUNCH without sync. */
enum { MSA_STEP_AUTO = 0, MSA_STEP_ONE_LAUNCH = 1, MSA_STEP_SEPARATE = 2 };
#define MSA_DECODE_STEP_SYNC_WORDS(rows, G) (4 + 2 * (int64_t)(rows) * (int64_t)(G))
msa_status_t msa_decode_step(const msa_dims_t *dims, int32_t rows, const void *q_idx,
                             msa_view_t k_idx, const int32_t *block_table, int32_t bt_stride,
                             const int32_t *row_req, const int32_t *row_pos,
                             const int32_t *blk_lo, int32_t num_reqs, int32_t score_stride,
                             int32_t k, const void *q, msa_view_t kc, msa_view_t vc,
                             float sm_scale, float *scores, int32_t *sel, int32_t *page_table,
                             void *o_part, float *lse_part, void *o, float *lse, int32_t *sync,
                             int32_t mode, msa_stream_t stream);

/* ------------------------------------------------------------------ f4
 * msa_gather_pages -- on-demand load of the selected KV pages.
 * Pages: future-work section (未来工作) of the aihot.news page: the CPU offload
 * of the key index and of the KV cache can be separated, the full key index
 * loaded and the KV cache loaded on demand from the top-k selection.
 *
 * For u = (r*G + g)*nslot + s and p = page_table[r][g][s] >= 0, copies the 128
 * tokens of page p, group g of k and of v (views, dim = D; typically pinned
 * host memory, see msa_view_t) to dst_k[u] and dst_v[u], and writes
 * dst_page_table[r][g][s] = u (-1 where p < 0).  msa_sparse_attn_decode then
 * reads the pool through the views {dst_k or dst_v, page_stride = 128*D,
 * group_stride = 0, token_stride = D} with dst_page_table, at device-memory
 * speed; the copy reads whole 256-byte token rows.
 *
 *   page_table      int32 [rows][G][nslot]
 *   dst_k, dst_v    device bf16 [rows*G*nslot][128][D], 16-byte aligned
 *   dst_page_table  device int32 [rows][G][nslot]
 * Errors: MSA_ERR_NULL, MSA_ERR_INVALID (alignment, sizes), MSA_ERR_UNSUPPORTED
 * (D != 128), MSA_ERR_HIP. */
msa_status_t msa_gather_pages(const msa_dims_t *dims, int32_t rows, const int32_t *page_table,
                              int32_t nslot, msa_view_t k, msa_view_t v, void *dst_k,
                              void *dst_v, int32_t *dst_page_table, msa_stream_t stream);

/* ------------------------------------------------------------------ a8 / a9
 * msa_sparse_attn_prefill -- KV-block-major sparse attention.
 * Pages: KV-block-major section (KV 块主序稀疏注意力): many queries select the
 * same KV block, so the {query, block} map is inverted into {block, queries}
 * and the block loop runs outside the query loop; every KV block is moved from
 * HBM once and yields partial outputs that a log-sum-exp reduction combines.
 *
 * Same inputs and outputs as msa_sparse_attn_decode (the results agree with it
 * up to fp32 summation order).  Internally it inverts sel into per-(group, page) query
 * lists in the workspace, then runs one pass per KV page that loads K and V
 * once and serves every (row, slot) that selected it.
 *
 *   num_pages   number of pages in the caches (page_table values < num_pages)
 *   workspace   device buffer of at least msa_prefill_workspace_size() bytes,
 *               16-byte aligned; contents on entry are ignored */
msa_status_t msa_prefill_workspace_size(const msa_dims_t *dims, int32_t rows, int32_t nslot,
                                        int32_t num_pages, size_t *bytes);

msa_status_t msa_sparse_attn_prefill(const msa_dims_t *dims, int32_t rows, const void *q,
                                     msa_view_t k, msa_view_t v, const int32_t *sel,
                                     const int32_t *page_table, int32_t nslot,
                                     const int32_t *row_pos, int32_t num_pages, float sm_scale,
                                     void *workspace, size_t workspace_bytes, void *o_part,
                                     float *lse_part, msa_stream_t stream);

/* ------------------------------------------------------------------ f3
 * msa_sparse_attn_prefill_merged -- msa_sparse_attn_prefill and msa_lse_merge
 * scheduled by query slabs.  Pages: KV-block-major section (KV 块主序稀疏注意力:
 * per-block partial outputs combined by a log-sum-exp reduction) and the fusion
 * of the q->kv remap named in 未来工作 of the aihot.news page.
 *
 * The rows are taken in slabs of slab_rows (0: all rows in one slab); for each
 * slab the q->kv inversion, the block-major attention and the merge run one
 * after the other, the slab's partials in the workspace, so the partials of a
 * slab are read back by its merge right after they are written (while they may
 * still sit in L2 / the last-level cache) and the caller never holds
 * rows x H x nslot partials.  Writes o (bf16 [rows][G*Hg][128], 16-byte aligned)
 * and lse (fp32 [rows][G*Hg], may be NULL): bit for bit what
 * msa_sparse_attn_prefill followed by msa_lse_merge write, for every slab size
 * (a partial depends only on its own row).  Smaller slabs hold fewer partials
 * but load each selected KV block once per slab that selects it.
 *
 *   slab_rows   >= 0; rows per slab (0 or >= rows: one slab)
 *   workspace   device buffer of at least msa_prefill_merged_workspace_size()
 *               bytes (same slab_rows), 256-byte aligned; contents ignored
 * Other arguments as msa_sparse_attn_prefill.  Errors: as that call;
 * MSA_ERR_WORKSPACE for a workspace smaller than needed. */
msa_status_t msa_prefill_merged_workspace_size(const msa_dims_t *dims, int32_t rows,
                                               int32_t nslot, int32_t num_pages,
                                               int32_t slab_rows, size_t *bytes);

msa_status_t msa_sparse_attn_prefill_merged(const msa_dims_t *dims, int32_t rows, const void *q,
                                            msa_view_t k, msa_view_t v, const int32_t *sel,
                                            const int32_t *page_table, int32_t nslot,
                                            const int32_t *row_pos, int32_t num_pages,
                                            float sm_scale, int32_t slab_rows, void *workspace,
                                            size_t workspace_bytes, void *o, float *lse,
                                            msa_stream_t stream);

/* ------------------------------------------------------------------ a8 / a9, no allocation
 * msa_sparse_attn_prefill_noalloc -- msa_sparse_attn_prefill for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid allocation): it takes no workspace and allocates nothing.
 *
 * Same arguments, results and errors as msa_sparse_attn_prefill without
 * workspace / workspace_bytes; the results are bit-identical to it.  The
 * workspace lives instead in a static device array of
 * MSA_NOALLOC_SCRATCH_BYTES bytes that each GPU the library runs on holds
 * until the process ends.  A call whose workspace
 * (msa_prefill_workspace_size) exceeds it fails with MSA_ERR_WORKSPACE before
 * anything is launched: 16 MiB covers e.g. 8,192 query rows x 8 groups x 17
 * slots on 544 pages (about 9 MB).  Nothing in the array needs to start
 * cleared; every call rewrites what it reads.  All calls on one GPU share its
 * array: calls that overlap in time on one GPU (concurrent streams, or
 * threads) race on it and must be serialised by the caller. */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

msa_status_t msa_sparse_attn_prefill_noalloc(const msa_dims_t *dims, int32_t rows,
                                             const void *q, msa_view_t k, msa_view_t v,
                                             const int32_t *sel, const int32_t *page_table,
                                             int32_t nslot, const int32_t *row_pos,
                                             int32_t num_pages, float sm_scale, void *o_part,
                                             float *lse_part, msa_stream_t stream);

/* ------------------------------------------------------------------ a5 / a10
 * msa_lse_merge -- log-sum-exp reduction of per-block partials.
 * Pages: the final reduction rescales the partial O outputs by their
 * log-sum-exp and sums them (KV 块主序稀疏注意力; the page's own formula did not
 * survive, this is the standard one):
 *     m = max_s lse_s,  w_s = exp(lse_s - m),
 *     o = sum_s w_s o_s / sum_s w_s,  lse = m + ln(sum_s w_s)
 * Slots with lse = -inf are skipped; a (row, head) with none gets o = 0 and
 * lse = -inf.
 *
 *   o_part  bf16 [rows][H][nslot][D];  lse_part fp32 [rows][nslot][H]
 *   o       bf16 [rows][H][D];         lse      fp32 [rows][H] (may be NULL)
 *   D must be 128. */
msa_status_t msa_lse_merge(int32_t rows, int32_t H, int32_t nslot, int32_t D,
                           const void *o_part, const float *lse_part, void *o, float *lse,
                           msa_stream_t stream);

/* ------------------------------------------------------------------ misc */
const char *msa_version(void);
const char *msa_status_string(msa_status_t s);
/* Thread-local description of the last error on this thread ("" if none). */
const char *msa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */

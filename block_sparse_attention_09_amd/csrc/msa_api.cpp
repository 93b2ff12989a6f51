// msa_api.cpp -- the extern "C" boundary of libmsa: argument validation,
// launch-geometry choice and status reporting.  No call synchronises or
// allocates; every kernel goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "msa.h"
#include "msa_internal.h"
#include "msa_peaks.h"

namespace {

thread_local std::string g_last_error;

msa_status_t fail(msa_status_t s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

msa_status_t ok() {
    g_last_error.clear();
    return MSA_OK;
}

msa_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, status, ...)                     \
    do {                                               \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

msa_status_t check_dims(const msa_dims_t *d, bool need_index, bool need_attn) {
    REQUIRE(d, MSA_ERR_NULL, "dims is NULL");
    REQUIRE(d->G >= 1, MSA_ERR_INVALID, "G = %d must be >= 1", d->G);
    REQUIRE(d->blk == msa::kBlk, MSA_ERR_UNSUPPORTED, "blk = %d: only 128-token blocks", d->blk);
    if (need_index) {
        REQUIRE(d->n_idx >= 1 && d->n_idx <= 16, MSA_ERR_UNSUPPORTED,
                "n_idx = %d: supported 1..16", d->n_idx);
        REQUIRE(d->d_idx == 64 || d->d_idx == 128, MSA_ERR_UNSUPPORTED,
                "d_idx = %d: supported 64 or 128", d->d_idx);
    }
    if (need_attn) {
        REQUIRE(d->D == 128, MSA_ERR_UNSUPPORTED, "D = %d: only head dimension 128", d->D);
        REQUIRE(d->Hg == 1 || d->Hg == 2 || d->Hg == 4 || d->Hg == 8 || d->Hg == 16,
                MSA_ERR_UNSUPPORTED, "Hg = %d: supported 1, 2, 4, 8, 16", d->Hg);
    }
    return MSA_OK;
}

msa_status_t check_view(const msa_view_t &v, const char *name) {
    REQUIRE(v.base, MSA_ERR_NULL, "%s.base is NULL", name);
    REQUIRE(aligned(v.base, 16), MSA_ERR_INVALID, "%s.base must be 16-byte aligned", name);
    REQUIRE(v.page_stride >= 0 && v.group_stride >= 0 && v.token_stride >= 0, MSA_ERR_INVALID,
            "%s strides must be >= 0", name);
    REQUIRE(v.page_stride % 8 == 0 && v.group_stride % 8 == 0 && v.token_stride % 8 == 0,
            MSA_ERR_INVALID, "%s strides must be multiples of 8 elements", name);
    return MSA_OK;
}

hipStream_t as_stream(msa_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// k and the selection size: k + 1 slots per (row, group) must stay far from
// int32 overflow (the kernels index slots and pad loops with int), and the
// whole selection rows * G * (k + 1) must fit an int32 element count.
msa_status_t check_k(int32_t k, int32_t rows, int32_t G) {
    REQUIRE(k >= 0 && k < (1 << 30), MSA_ERR_INVALID, "k = %d must be in [0, 2^30)", k);
    REQUIRE((int64_t)rows * G * ((int64_t)k + 1) < (int64_t)INT32_MAX, MSA_ERR_INVALID,
            "rows * G * (k + 1) = %lld must fit in int32",
            (long long)((int64_t)rows * G * ((int64_t)k + 1)));
    return MSA_OK;
}

}  // namespace

extern "C" {

const char *msa_version(void) { return "libmsa 0.1.0 (gfx950)"; }

const char *msa_last_error(void) { return g_last_error.c_str(); }

const char *msa_status_string(msa_status_t s) {
    switch (s) {
        case MSA_OK: return "MSA_OK";
        case MSA_ERR_NULL: return "MSA_ERR_NULL: a required pointer is NULL";
        case MSA_ERR_INVALID: return "MSA_ERR_INVALID: invalid size, stride or alignment";
        case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: shape not supported";
        case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE: workspace too small";
        case MSA_ERR_HIP: return "MSA_ERR_HIP: HIP launch failed";
    }
    return "unknown msa_status_t";
}

msa_status_t msa_index_score(const msa_dims_t *dims, int32_t rows, const void *q_idx,
                             msa_view_t k_idx, const int32_t *block_table, int32_t bt_stride,
                             const int32_t *row_req, const int32_t *row_pos,
                             const int32_t *blk_lo, int32_t num_reqs, float *scores,
                             int32_t score_stride, msa_stream_t stream) {
    msa_status_t st = check_dims(dims, true, false);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0, MSA_ERR_INVALID, "rows = %d must be >= 0", rows);
    REQUIRE(score_stride >= 1, MSA_ERR_INVALID, "score_stride = %d must be >= 1", score_stride);
    REQUIRE(bt_stride >= 1, MSA_ERR_INVALID, "bt_stride = %d must be >= 1", bt_stride);
    REQUIRE(num_reqs >= 1, MSA_ERR_INVALID, "num_reqs = %d must be >= 1", num_reqs);
    if (rows == 0) return ok();
    REQUIRE(q_idx && block_table && row_pos && scores, MSA_ERR_NULL,
            "q_idx, block_table, row_pos and scores are required");
    REQUIRE(aligned(q_idx, 16), MSA_ERR_INVALID, "q_idx must be 16-byte aligned");
    REQUIRE(aligned(scores, 4) && aligned(block_table, 4) && aligned(row_pos, 4), MSA_ERR_INVALID,
            "int32/fp32 arrays must be 4-byte aligned");
    st = check_view(k_idx, "k_idx");
    if (st != MSA_OK) return st;
    return hip_status(msa::launch_index_score(*dims, rows, static_cast<const msa::bf16_t *>(q_idx),
                                              k_idx, block_table, bt_stride, row_req, row_pos,
                                              blk_lo, num_reqs, scores, score_stride,
                                              as_stream(stream)),
                      "msa_index_score");
}

msa_status_t msa_topk_blocks(const msa_dims_t *dims, int32_t rows, const float *scores,
                             int32_t score_stride, const int32_t *row_pos, int32_t k,
                             int32_t *sel, msa_stream_t stream) {
    msa_status_t st = check_dims(dims, false, false);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0, MSA_ERR_INVALID, "rows = %d must be >= 0", rows);
    if ((st = check_k(k, rows, dims->G)) != MSA_OK) return st;
    REQUIRE(score_stride >= 1, MSA_ERR_INVALID, "score_stride = %d must be >= 1", score_stride);
    if (rows == 0) return ok();
    REQUIRE(scores && row_pos && sel, MSA_ERR_NULL, "scores, row_pos and sel are required");
    return hip_status(msa::launch_topk(rows, dims->G, scores, score_stride, row_pos, k, sel,
                                       as_stream(stream)),
                      "msa_topk_blocks");
}

msa_status_t msa_topk_blocks_paged(const msa_dims_t *dims, int32_t rows, const float *scores,
                                   int32_t score_stride, const int32_t *row_pos, int32_t k,
                                   const int32_t *row_req, const int32_t *block_table,
                                   int32_t bt_stride, int32_t *sel, int32_t *page_table,
                                   msa_stream_t stream) {
    msa_status_t st = check_dims(dims, false, false);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0, MSA_ERR_INVALID, "rows = %d must be >= 0", rows);
    if ((st = check_k(k, rows, dims->G)) != MSA_OK) return st;
    REQUIRE(score_stride >= 1, MSA_ERR_INVALID, "score_stride = %d must be >= 1", score_stride);
    REQUIRE(bt_stride >= 1, MSA_ERR_INVALID, "bt_stride = %d must be >= 1", bt_stride);
    if (rows == 0) return ok();
    REQUIRE(scores && row_pos && sel && block_table && page_table, MSA_ERR_NULL,
            "scores, row_pos, block_table, sel and page_table are required");
    return hip_status(msa::launch_topk(rows, dims->G, scores, score_stride, row_pos, k, sel,
                                       as_stream(stream), row_req, block_table, bt_stride,
                                       page_table),
                      "msa_topk_blocks_paged");
}

msa_status_t msa_build_page_table(const msa_dims_t *dims, int32_t rows, const int32_t *sel,
                                  int32_t nslot, const int32_t *row_req,
                                  const int32_t *block_table, int32_t bt_stride,
                                  int32_t *page_table, msa_stream_t stream) {
    msa_status_t st = check_dims(dims, false, false);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0, MSA_ERR_INVALID, "rows = %d must be >= 0", rows);
    REQUIRE(nslot >= 1, MSA_ERR_INVALID, "nslot = %d must be >= 1", nslot);
    REQUIRE(bt_stride >= 1, MSA_ERR_INVALID, "bt_stride = %d must be >= 1", bt_stride);
    if (rows == 0) return ok();
    REQUIRE(sel && block_table && page_table, MSA_ERR_NULL,
            "sel, block_table and page_table are required");
    return hip_status(msa::launch_page_table(rows, dims->G, sel, nslot, row_req, block_table,
                                             bt_stride, page_table, as_stream(stream)),
                      "msa_build_page_table");
}

static msa_status_t check_attn(const msa_dims_t *dims, int32_t rows, const void *q,
                               const msa_view_t &k, const msa_view_t &v, const int32_t *sel,
                               const int32_t *page_table, int32_t nslot, const int32_t *row_pos,
                               float sm_scale, const void *o_part, const float *lse_part) {
    msa_status_t st = check_dims(dims, false, true);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0, MSA_ERR_INVALID, "rows = %d must be >= 0", rows);
    REQUIRE(nslot >= 1, MSA_ERR_INVALID, "nslot = %d must be >= 1", nslot);
    REQUIRE(std::isfinite(sm_scale) && sm_scale > 0.f, MSA_ERR_INVALID,
            "sm_scale must be finite and > 0");
    REQUIRE((int64_t)rows * nslot < (int64_t)1 << 31, MSA_ERR_INVALID,
            "rows * nslot must fit in int32");
    if (rows == 0) return MSA_OK;
    REQUIRE(q && sel && page_table && row_pos && o_part && lse_part, MSA_ERR_NULL,
            "q, sel, page_table, row_pos, o_part and lse_part are required");
    REQUIRE(aligned(q, 16) && aligned(o_part, 16), MSA_ERR_INVALID,
            "q and o_part must be 16-byte aligned");
    st = check_view(k, "k");
    if (st != MSA_OK) return st;
    return check_view(v, "v");
}

static msa::AttnArgs attn_args(const msa_dims_t *d, int32_t rows, const void *q,
                               const msa_view_t &k, const msa_view_t &v, const int32_t *sel,
                               const int32_t *pt, int32_t nslot, const int32_t *row_pos,
                               float sm_scale, void *o_part, float *lse_part) {
    msa::AttnArgs a;
    a.rows = rows;
    a.G = d->G;
    a.Hg = d->Hg;
    a.nslot = nslot;
    a.q = static_cast<const msa::bf16_t *>(q);
    a.k = static_cast<const msa::bf16_t *>(k.base);
    a.kps = k.page_stride;
    a.kgs = k.group_stride;
    a.kts = k.token_stride;
    a.v = static_cast<const msa::bf16_t *>(v.base);
    a.vps = v.page_stride;
    a.vgs = v.group_stride;
    a.vts = v.token_stride;
    a.sel = sel;
    a.page_table = pt;
    a.row_pos = row_pos;
    a.sm_scale = sm_scale;
    a.o_part = static_cast<msa::bf16_t *>(o_part);
    a.lse_part = lse_part;
    return a;
}

msa_status_t msa_sparse_attn_decode(const msa_dims_t *dims, int32_t rows, const void *q,
                                    msa_view_t k, msa_view_t v, const int32_t *sel,
                                    const int32_t *page_table, int32_t nslot,
                                    const int32_t *row_pos, float sm_scale, void *o_part,
                                    float *lse_part, msa_stream_t stream) {
    msa_status_t st = check_attn(dims, rows, q, k, v, sel, page_table, nslot, row_pos, sm_scale,
                                 o_part, lse_part);
    if (st != MSA_OK) return st;
    if (rows == 0) return ok();
    const msa::AttnArgs a =
        attn_args(dims, rows, q, k, v, sel, page_table, nslot, row_pos, sm_scale, o_part, lse_part);
    return hip_status(msa::launch_attn_decode(a, as_stream(stream)), "msa_sparse_attn_decode");
}

// Selection, page table and decode attention (validated arguments): one kernel
// when its grid runs in a single round -- every workgroup repeats its group's
// top-k, which costs nothing extra while all of them run at once but would be
// paid again by every later round of a larger batch -- else top-k, then
// attention.
static hipError_t decode_select(const msa::AttnArgs &a, const float *scores, int32_t score_stride,
                                int32_t k, const int32_t *row_req, const int32_t *block_table,
                                int32_t bt_stride, int32_t *sel, int32_t *page_table,
                                hipStream_t stream) {
    const int64_t units = (int64_t)a.rows * a.G * a.nslot;
    if (score_stride <= msa::kSelectMaxBlocks && units <= msa::decode_select_capacity(a.Hg)) {
        const msa::SelectArgs sa{scores, score_stride, k,   row_req,
                                 block_table, bt_stride, sel, page_table};
        return msa::launch_attn_decode_select(a, sa, stream);
    }
    hipError_t e = msa::launch_topk(a.rows, a.G, scores, score_stride, a.row_pos, k, sel, stream,
                                    row_req, block_table, bt_stride, page_table);
    if (e == hipSuccess) e = msa::launch_attn_decode(a, stream);
    return e;
}

msa_status_t msa_sparse_attn_decode_select(const msa_dims_t *dims, int32_t rows,
                                           const float *scores, int32_t score_stride, int32_t k,
                                           const int32_t *row_req, const int32_t *block_table,
                                           int32_t bt_stride, const void *q, msa_view_t kc,
                                           msa_view_t vc, const int32_t *row_pos, float sm_scale,
                                           int32_t *sel, int32_t *page_table, void *o_part,
                                           float *lse_part, msa_stream_t stream) {
    REQUIRE(dims, MSA_ERR_NULL, "dims is NULL");
    REQUIRE(rows >= 0, MSA_ERR_INVALID, "rows = %d must be >= 0", rows);
    msa_status_t st = check_k(k, rows, dims->G);
    if (st != MSA_OK) return st;
    REQUIRE(score_stride >= 1, MSA_ERR_INVALID, "score_stride = %d must be >= 1", score_stride);
    REQUIRE(bt_stride >= 1, MSA_ERR_INVALID, "bt_stride = %d must be >= 1", bt_stride);
    const int32_t nslot = k + 1;
    st = check_attn(dims, rows, q, kc, vc, sel, page_table, nslot, row_pos,
                                 sm_scale, o_part, lse_part);
    if (st != MSA_OK) return st;
    if (rows == 0) return ok();
    REQUIRE(scores && block_table, MSA_ERR_NULL, "scores and block_table are required");
    const msa::AttnArgs a = attn_args(dims, rows, q, kc, vc, sel, page_table, nslot, row_pos,
                                      sm_scale, o_part, lse_part);
    return hip_status(decode_select(a, scores, score_stride, k, row_req, block_table, bt_stride,
                                    sel, page_table, as_stream(stream)),
                      "msa_sparse_attn_decode_select");
}

msa_status_t msa_decode_step(const msa_dims_t *dims, int32_t rows, const void *q_idx,
                             msa_view_t k_idx, const int32_t *block_table, int32_t bt_stride,
                             const int32_t *row_req, const int32_t *row_pos,
                             const int32_t *blk_lo, int32_t num_reqs, int32_t score_stride,
                             int32_t k, const void *q, msa_view_t kc, msa_view_t vc,
                             float sm_scale, float *scores, int32_t *sel, int32_t *page_table,
                             void *o_part, float *lse_part, void *o, float *lse, int32_t *sync,
                             int32_t mode, msa_stream_t stream) {
    msa_status_t st = check_dims(dims, true, true);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0, MSA_ERR_INVALID, "rows = %d must be >= 0", rows);
    REQUIRE(mode == MSA_STEP_AUTO || mode == MSA_STEP_ONE_LAUNCH || mode == MSA_STEP_SEPARATE,
            MSA_ERR_INVALID, "mode = %d: MSA_STEP_AUTO, MSA_STEP_ONE_LAUNCH or MSA_STEP_SEPARATE",
            mode);
    REQUIRE(score_stride >= 1, MSA_ERR_INVALID, "score_stride = %d must be >= 1", score_stride);
    REQUIRE(bt_stride >= 1, MSA_ERR_INVALID, "bt_stride = %d must be >= 1", bt_stride);
    REQUIRE(num_reqs >= 1, MSA_ERR_INVALID, "num_reqs = %d must be >= 1", num_reqs);
    if ((st = check_k(k, rows, dims->G)) != MSA_OK) return st;
    const int32_t nslot = k + 1;
    st = check_attn(dims, rows, q, kc, vc, sel, page_table, nslot, row_pos, sm_scale, o_part,
                    lse_part);
    if (st != MSA_OK) return st;
    const bool supported = msa::decode_step_supported(dims->d_idx, score_stride);
    REQUIRE(mode != MSA_STEP_ONE_LAUNCH || supported, MSA_ERR_UNSUPPORTED,
            "MSA_STEP_ONE_LAUNCH needs score_stride <= %d", msa::kSelectMaxBlocks);
    REQUIRE(mode != MSA_STEP_ONE_LAUNCH || sync, MSA_ERR_NULL,
            "MSA_STEP_ONE_LAUNCH needs the sync words");
    REQUIRE((int64_t)rows * dims->G < ((int64_t)1 << 28), MSA_ERR_INVALID,
            "rows * G must be below 2^28");
    if (rows == 0) return ok();
    REQUIRE(q_idx && block_table && scores && o, MSA_ERR_NULL,
            "q_idx, block_table, scores and o are required");
    REQUIRE(aligned(q_idx, 16) && aligned(o, 16), MSA_ERR_INVALID,
            "q_idx and o must be 16-byte aligned");
    REQUIRE(aligned(scores, 4) && aligned(block_table, 4) && aligned(row_pos, 4) &&
                aligned(sync, 4),
            MSA_ERR_INVALID, "int32/fp32 arrays must be 4-byte aligned");
    if ((st = check_view(k_idx, "k_idx")) != MSA_OK) return st;
    // the automatic mode takes the separate launches: on MI355X they are the
    // faster form at every decode shape measured (issued back to back, the
    // three kernels' launch gaps cost less than the single launch's fences and
    // waits: 21.2 against 25.1 us at a 4K context, 196 against 415 us at
    // batch 8 x 64K)
    const bool one = supported && mode == MSA_STEP_ONE_LAUNCH;
    const msa::AttnArgs a = attn_args(dims, rows, q, kc, vc, sel, page_table, nslot, row_pos,
                                      sm_scale, o_part, lse_part);
    const hipStream_t s = as_stream(stream);
    if (one) {
        msa::StepArgs f{};
        f.n_idx = dims->n_idx;
        f.q_idx = static_cast<const msa::bf16_t *>(q_idx);
        f.kidx = static_cast<const msa::bf16_t *>(k_idx.base);
        f.kips = k_idx.page_stride;
        f.kigs = k_idx.group_stride;
        f.kits = k_idx.token_stride;
        f.block_table = block_table;
        f.bt_stride = bt_stride;
        f.row_req = row_req;
        f.blk_lo = blk_lo;
        f.scores = scores;
        f.score_stride = score_stride;
        f.k = k;
        f.sel = sel;
        f.page_table = page_table;
        f.o = static_cast<msa::bf16_t *>(o);
        f.lse = lse;
        f.index_scale = 1.0f / sqrtf((float)dims->d_idx);
        f.sync = sync;
        return hip_status(msa::launch_decode_step(a, f, dims->d_idx, s), "msa_decode_step");
    }
    hipError_t e = msa::launch_index_score(*dims, rows, static_cast<const msa::bf16_t *>(q_idx),
                                           k_idx, block_table, bt_stride, row_req, row_pos,
                                           blk_lo, num_reqs, scores, score_stride, s);
    if (e == hipSuccess)
        e = decode_select(a, scores, score_stride, k, row_req, block_table, bt_stride, sel,
                          page_table, s);
    if (e == hipSuccess)
        e = msa::launch_lse_merge(rows, dims->G * dims->Hg, nslot, a.o_part, lse_part,
                                  static_cast<msa::bf16_t *>(o), lse, s);
    return hip_status(e, "msa_decode_step");
}

msa_status_t msa_prefill_workspace_size(const msa_dims_t *dims, int32_t rows, int32_t nslot,
                                        int32_t num_pages, size_t *bytes) {
    REQUIRE(bytes, MSA_ERR_NULL, "bytes is NULL");
    msa_status_t st = check_dims(dims, false, true);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0 && nslot >= 1 && num_pages >= 1, MSA_ERR_INVALID,
            "rows >= 0, nslot >= 1 and num_pages >= 1 are required");
    *bytes = msa::prefill_workspace_bytes(rows, dims->G, nslot, num_pages);
    return ok();
}

msa_status_t msa_sparse_attn_prefill(const msa_dims_t *dims, int32_t rows, const void *q,
                                     msa_view_t k, msa_view_t v, const int32_t *sel,
                                     const int32_t *page_table, int32_t nslot,
                                     const int32_t *row_pos, int32_t num_pages, float sm_scale,
                                     void *workspace, size_t workspace_bytes, void *o_part,
                                     float *lse_part, msa_stream_t stream) {
    msa_status_t st = check_attn(dims, rows, q, k, v, sel, page_table, nslot, row_pos, sm_scale,
                                 o_part, lse_part);
    if (st != MSA_OK) return st;
    REQUIRE(num_pages >= 1, MSA_ERR_INVALID, "num_pages = %d must be >= 1", num_pages);
    REQUIRE((int64_t)dims->G * num_pages < ((int64_t)1 << 31) - 1, MSA_ERR_INVALID,
            "G * num_pages must fit in int32");
    if (rows == 0) return ok();
    const size_t need = msa::prefill_workspace_bytes(rows, dims->G, nslot, num_pages);
    REQUIRE(workspace, MSA_ERR_NULL, "workspace is NULL");
    REQUIRE(aligned(workspace, 16), MSA_ERR_INVALID, "workspace must be 16-byte aligned");
    REQUIRE(workspace_bytes >= need, MSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu",
            workspace_bytes, need);
    const msa::AttnArgs a =
        attn_args(dims, rows, q, k, v, sel, page_table, nslot, row_pos, sm_scale, o_part, lse_part);
    return hip_status(msa::launch_attn_prefill(a, num_pages, workspace, as_stream(stream)),
                      "msa_sparse_attn_prefill");
}

msa_status_t msa_sparse_attn_prefill_noalloc(const msa_dims_t *dims, int32_t rows,
                                             const void *q, msa_view_t k, msa_view_t v,
                                             const int32_t *sel, const int32_t *page_table,
                                             int32_t nslot, const int32_t *row_pos,
                                             int32_t num_pages, float sm_scale, void *o_part,
                                             float *lse_part, msa_stream_t stream) {
    msa_status_t st = check_attn(dims, rows, q, k, v, sel, page_table, nslot, row_pos, sm_scale,
                                 o_part, lse_part);
    if (st != MSA_OK) return st;
    REQUIRE(num_pages >= 1, MSA_ERR_INVALID, "num_pages = %d must be >= 1", num_pages);
    REQUIRE((int64_t)dims->G * num_pages < ((int64_t)1 << 31) - 1, MSA_ERR_INVALID,
            "G * num_pages must fit in int32");
    if (rows == 0) return ok();
    const size_t need = msa::prefill_workspace_bytes(rows, dims->G, nslot, num_pages);
    REQUIRE(need <= msa::kNoallocScratchBytes, MSA_ERR_WORKSPACE,
            "this prefill needs %zu bytes of workspace, beyond the %zu-byte static scratch of "
            "the allocation-free call (use msa_sparse_attn_prefill with a workspace)",
            need, msa::kNoallocScratchBytes);
    void *ws = nullptr;
    const hipError_t e = msa::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "msa_sparse_attn_prefill_noalloc: scratch address");
    const msa::AttnArgs a =
        attn_args(dims, rows, q, k, v, sel, page_table, nslot, row_pos, sm_scale, o_part, lse_part);
    return hip_status(msa::launch_attn_prefill(a, num_pages, ws, as_stream(stream)),
                      "msa_sparse_attn_prefill_noalloc");
}

// Workspace of the slab-scheduled prefill: the remap of one slab, then the
// slab's partial outputs and LSEs.
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
struct SlabLayout {
    size_t remap, part, lse, total;
};
static SlabLayout slab_layout(const msa_dims_t *d, int32_t slab, int32_t nslot, int32_t num_pages) {
    SlabLayout L;
    const size_t H = (size_t)d->G * d->Hg;
    L.remap = align256(msa::prefill_workspace_bytes(slab, d->G, nslot, num_pages));
    L.part = align256((size_t)slab * H * nslot * 128 * sizeof(uint16_t));
    L.lse = align256((size_t)slab * H * nslot * sizeof(float));
    L.total = L.remap + L.part + L.lse;
    return L;
}

msa_status_t msa_prefill_merged_workspace_size(const msa_dims_t *dims, int32_t rows,
                                               int32_t nslot, int32_t num_pages,
                                               int32_t slab_rows, size_t *bytes) {
    REQUIRE(bytes, MSA_ERR_NULL, "bytes is NULL");
    msa_status_t st = check_dims(dims, false, true);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0 && nslot >= 1 && num_pages >= 1 && slab_rows >= 0, MSA_ERR_INVALID,
            "rows >= 0, nslot >= 1, num_pages >= 1 and slab_rows >= 0 are required");
    const int32_t slab = (slab_rows == 0 || slab_rows > rows) ? rows : slab_rows;
    *bytes = slab_layout(dims, slab, nslot, num_pages).total;
    return ok();
}

msa_status_t msa_sparse_attn_prefill_merged(const msa_dims_t *dims, int32_t rows, const void *q,
                                            msa_view_t k, msa_view_t v, const int32_t *sel,
                                            const int32_t *page_table, int32_t nslot,
                                            const int32_t *row_pos, int32_t num_pages,
                                            float sm_scale, int32_t slab_rows, void *workspace,
                                            size_t workspace_bytes, void *o, float *lse,
                                            msa_stream_t stream) {
    // the partials live in the workspace: check_attn's o_part / lse_part
    // requirements are met by the workspace checks below
    msa_status_t st = check_attn(dims, rows, q, k, v, sel, page_table, nslot, row_pos, sm_scale,
                                 workspace, static_cast<const float *>(workspace));
    if (st != MSA_OK) return st;
    REQUIRE(num_pages >= 1, MSA_ERR_INVALID, "num_pages = %d must be >= 1", num_pages);
    REQUIRE((int64_t)dims->G * num_pages < ((int64_t)1 << 31) - 1, MSA_ERR_INVALID,
            "G * num_pages must fit in int32");
    REQUIRE(slab_rows >= 0, MSA_ERR_INVALID, "slab_rows = %d must be >= 0", slab_rows);
    if (rows == 0) return ok();
    REQUIRE(o, MSA_ERR_NULL, "o is required");
    REQUIRE(aligned(o, 16), MSA_ERR_INVALID, "o must be 16-byte aligned");
    const int32_t slab = (slab_rows == 0 || slab_rows > rows) ? rows : slab_rows;
    const SlabLayout L = slab_layout(dims, slab, nslot, num_pages);
    REQUIRE(aligned(workspace, 256), MSA_ERR_INVALID, "workspace must be 256-byte aligned");
    REQUIRE(workspace_bytes >= L.total, MSA_ERR_WORKSPACE, "workspace of %zu bytes, need %zu",
            workspace_bytes, L.total);
    char *ws = static_cast<char *>(workspace);
    void *part = ws + L.remap;
    float *lse_part = reinterpret_cast<float *>(ws + L.remap + L.part);
    const int H = dims->G * dims->Hg;
    const hipStream_t s = as_stream(stream);
    for (int32_t r0 = 0; r0 < rows; r0 += slab) {
        const int32_t n = std::min(slab, rows - r0);
        const size_t sl = (size_t)r0 * dims->G * nslot;
        const msa::AttnArgs a = attn_args(
            dims, n, static_cast<const msa::bf16_t *>(q) + (size_t)r0 * H * 128, k, v, sel + sl,
            page_table + sl, nslot, row_pos + r0, sm_scale, part, lse_part);
        hipError_t e = msa::launch_attn_prefill(a, num_pages, ws, s);
        if (e == hipSuccess)
            e = msa::launch_lse_merge(n, H, nslot, static_cast<const msa::bf16_t *>(part),
                                      lse_part, static_cast<msa::bf16_t *>(o) + (size_t)r0 * H * 128,
                                      lse ? lse + (size_t)r0 * H : nullptr, s);
        if (e != hipSuccess) return hip_status(e, "msa_sparse_attn_prefill_merged");
    }
    return ok();
}

msa_status_t msa_lse_merge(int32_t rows, int32_t H, int32_t nslot, int32_t D, const void *o_part,
                           const float *lse_part, void *o, float *lse, msa_stream_t stream) {
    REQUIRE(rows >= 0 && H >= 1 && nslot >= 1, MSA_ERR_INVALID,
            "rows >= 0, H >= 1 and nslot >= 1 are required");
    REQUIRE(D == 128, MSA_ERR_UNSUPPORTED, "D = %d: only head dimension 128", D);
    if (rows == 0) return ok();
    REQUIRE(o_part && lse_part && o, MSA_ERR_NULL, "o_part, lse_part and o are required");
    REQUIRE(aligned(o_part, 16) && aligned(o, 16), MSA_ERR_INVALID,
            "o_part and o must be 16-byte aligned");
    return hip_status(msa::launch_lse_merge(rows, H, nslot, static_cast<const msa::bf16_t *>(o_part),
                                            lse_part, static_cast<msa::bf16_t *>(o), lse,
                                            as_stream(stream)),
                      "msa_lse_merge");
}

msa_status_t msa_gather_pages(const msa_dims_t *dims, int32_t rows, const int32_t *page_table,
                              int32_t nslot, msa_view_t k, msa_view_t v, void *dst_k,
                              void *dst_v, int32_t *dst_page_table, msa_stream_t stream) {
    msa_status_t st = check_dims(dims, false, true);
    if (st != MSA_OK) return st;
    REQUIRE(rows >= 0 && nslot >= 1, MSA_ERR_INVALID, "rows >= 0 and nslot >= 1 are required");
    if (rows == 0) return ok();
    REQUIRE(page_table && dst_k && dst_v && dst_page_table, MSA_ERR_NULL,
            "page_table, dst_k, dst_v and dst_page_table are required");
    if ((st = check_view(k, "k")) != MSA_OK) return st;
    if ((st = check_view(v, "v")) != MSA_OK) return st;
    REQUIRE(aligned(dst_k, 16) && aligned(dst_v, 16), MSA_ERR_INVALID,
            "dst_k and dst_v must be 16-byte aligned");
    REQUIRE((int64_t)rows * dims->G * nslot < (int64_t)INT32_MAX, MSA_ERR_INVALID,
            "rows * G * nslot must fit in int32 (the pool's page ids)");
    return hip_status(msa::launch_gather_pages(rows, dims->G, nslot, page_table, k, v,
                                               static_cast<msa::bf16_t *>(dst_k),
                                               static_cast<msa::bf16_t *>(dst_v), dst_page_table,
                                               as_stream(stream)),
                      "msa_gather_pages");
}

msa_status_t msa_peak_stream_read(const void *buf, size_t bytes, float *sink,
                                  msa_stream_t stream) {
    REQUIRE(bytes % 16 == 0, MSA_ERR_INVALID, "bytes = %zu must be a multiple of 16", bytes);
    if (bytes == 0) return ok();
    REQUIRE(buf && sink, MSA_ERR_NULL, "buf and sink are required");
    REQUIRE(aligned(buf, 16), MSA_ERR_INVALID, "buf must be 16-byte aligned");
    return hip_status(msa::launch_peak_stream_read(buf, (int64_t)bytes, sink, as_stream(stream)),
                      "msa_peak_stream_read");
}

msa_status_t msa_peak_stream_write(void *buf, size_t bytes, uint32_t tag, msa_stream_t stream) {
    REQUIRE(bytes % 16 == 0, MSA_ERR_INVALID, "bytes = %zu must be a multiple of 16", bytes);
    if (bytes == 0) return ok();
    REQUIRE(buf, MSA_ERR_NULL, "buf is required");
    REQUIRE(aligned(buf, 16), MSA_ERR_INVALID, "buf must be 16-byte aligned");
    return hip_status(msa::launch_peak_stream_write(buf, (int64_t)bytes, tag, as_stream(stream)),
                      "msa_peak_stream_write");
}

msa_status_t msa_peak_row_copy(const void *src, void *dst, const int32_t *load_idx,
                               const int32_t *store_idx, int64_t n, int32_t tiles_per_wg,
                               int32_t load_layout, msa_stream_t stream) {
    REQUIRE(n >= 0 && n % 32 == 0, MSA_ERR_INVALID, "n = %lld must be a multiple of 32 (>= 0)",
            (long long)n);
    REQUIRE(tiles_per_wg >= 1 && tiles_per_wg <= 64, MSA_ERR_INVALID,
            "tiles_per_wg = %d must be in [1, 64]", tiles_per_wg);
    REQUIRE(load_layout == 0 || load_layout == 1, MSA_ERR_INVALID,
            "load_layout = %d must be 0 or 1", load_layout);
    REQUIRE(n / 32 / tiles_per_wg < ((int64_t)1 << 31), MSA_ERR_INVALID, "n too large");
    if (n == 0) return ok();
    REQUIRE(src && dst && load_idx && store_idx, MSA_ERR_NULL,
            "src, dst, load_idx and store_idx are required");
    REQUIRE(aligned(src, 16) && aligned(dst, 16) && aligned(load_idx, 4) && aligned(store_idx, 4),
            MSA_ERR_INVALID, "src and dst must be 16-byte aligned, the indices 4-byte aligned");
    return hip_status(msa::launch_peak_row_copy(src, dst, load_idx, store_idx, n, tiles_per_wg,
                                                load_layout, as_stream(stream)),
                      "msa_peak_row_copy");
}

msa_status_t msa_peak_mfma_bf16(int32_t iters, float *sink, double *flops, msa_stream_t stream) {
    REQUIRE(iters >= 1, MSA_ERR_INVALID, "iters = %d must be >= 1", iters);
    REQUIRE(sink && flops, MSA_ERR_NULL, "sink and flops are required");
    return hip_status(msa::launch_peak_mfma_bf16(iters, sink, flops, as_stream(stream)),
                      "msa_peak_mfma_bf16");
}

msa_status_t msa_peak_mfma_bf16_random(int32_t iters, float *sink, double *flops,
                                       msa_stream_t stream) {
    REQUIRE(iters >= 1, MSA_ERR_INVALID, "iters = %d must be >= 1", iters);
    REQUIRE(sink && flops, MSA_ERR_NULL, "sink and flops are required");
    return hip_status(msa::launch_peak_mfma_bf16_random(iters, sink, flops, as_stream(stream)),
                      "msa_peak_mfma_bf16_random");
}

}  // extern "C"

// index_score_tiled.hip -- block scores for the prefill shape (gfx950).
//
// Pages: decode index-scoring section (解码索引评分内核优化) of "Together AI 解析如何
// 高效服务 MiniMax M3" defines the scan; in a prefill chunk many query rows of one
// request score the same key pages, so the key index is shared across a tile of
// rows here instead of streamed once per row.  Same score as the streaming
// kernel: max over visible tokens t of qbar . k_t / sqrt(d_idx), qbar = sum_j q_j
// in fp32 split into bf16 hi + lo for two MFMA passes.
#include "msa_internal.h"

namespace msa {

namespace {

// Tiled kernel (prefill shape: many rows of one request share every key page).
// A workgroup owns 128 consecutive rows and one KV group and walks the blocks
// of the rows' request: each 128-token key block is staged once in LDS (double
// buffered, the next block's global loads in flight during the current block's
// MFMAs) and serves all 128 rows, so the key index is read once per row tile
// instead of once per row.  Wave w owns rows 32w .. 32w+31 (two 16-row MFMA N
// tiles with qbar hi/lo in registers) against all 8 token tiles of the block.
// Rows of different requests in one tile are served in separate runs.
// Workgroup id = tile * G + g, so with the default round-robin dispatch over
// the 8 XCDs all tiles of one group share an XCD's L2 and walk the same key
// pages in step.
constexpr int kTileRows = 128;

template <int DIDX>
__global__ __launch_bounds__(256, 2) void index_score_tiled_kernel(
    int rows, int G, int n_idx, const bf16_t *__restrict__ q_idx, const bf16_t *__restrict__ kbase,
    int64_t kps, int64_t kgs, int64_t kts, const int32_t *__restrict__ block_table, int bt_stride,
    const int32_t *__restrict__ row_req, const int32_t *__restrict__ row_pos,
    const int32_t *__restrict__ blk_lo, float *__restrict__ scores, int score_stride, float scale) {
    constexpr int KST = DIDX + 16;     // LDS row stride of a staged block (32-B pad: conflict-free fragment reads)
    constexpr int NC = DIDX / 32;      // MFMA K chunks
    constexpr int LD_PER_THREAD = kBlk * DIDX / 8 / 256;   // 16-B loads per thread per block
    __shared__ __attribute__((aligned(16))) bf16_t kbuf[2][kBlk * KST];
    __shared__ int s_req[kTileRows], s_pos[kTileRows], s_slo[kTileRows];
    __shared__ int s_run[5];  // request, first and last block, unmasked block range

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = blockIdx.x % G;
    const int row0 = (blockIdx.x / G) * kTileRows;
    const int nrows = min(kTileRows, rows - row0);

    if (tid < kTileRows) {
        int req = -1, pos = -1, slo = 0;
        if (tid < nrows) {
            const int r = row0 + tid;
            req = row_req ? row_req[r] : r;
            pos = row_pos[r];
            const int own = pos / kBlk;
            const int lo = blk_lo ? blk_lo[(int64_t)req * G + g] : 0;
            slo = lo < own ? lo : own;
        }
        s_req[tid] = req;
        s_pos[tid] = pos;
        s_slo[tid] = slo;
    }
    __syncthreads();
    // -inf for every block outside a row's scored range [slo, own]
    for (int i = 0; i < nrows; ++i) {
        const int own = s_pos[i] / kBlk, slo = s_slo[i];
        float *out = scores + ((int64_t)(row0 + i) * G + g) * score_stride;
        for (int b = tid; b < score_stride; b += 256)
            if (b < slo || b > own) out[b] = -INFINITY;
    }

    // qbar hi/lo B fragments of this wave's 32 rows
    const int kq = (lane >> 4) * 8;
    bf16x8 bhi[2][NC], blo[2][NC];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int i = 32 * w + 16 * nt + (lane & 15);
        float acc[NC][8];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
        if (i < nrows) {
            const bf16_t *qb = q_idx + ((int64_t)(row0 + i) * G + g) * n_idx * DIDX + kq;
            for (int j0 = 0; j0 < n_idx; j0 += 4) {
                u32x4 wv[4][NC];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        wv[jj][c] = (j0 + jj < n_idx) ? ld16(qb + (j0 + jj) * DIDX + 32 * c)
                                                      : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            acc[c][2 * e] += bf16_lo(wv[jj][c][e]);
                            acc[c][2 * e + 1] += bf16_hi(wv[jj][c][e]);
                        }
            }
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            u32x4 hw, lw;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t h0 = f32_to_bf16_rne(acc[c][2 * e]);
                const uint32_t h1 = f32_to_bf16_rne(acc[c][2 * e + 1]);
                hw[e] = h0 | (h1 << 16);
                lw[e] = f32_to_bf16_rne(acc[c][2 * e] - __uint_as_float(h0 << 16)) |
                        (f32_to_bf16_rne(acc[c][2 * e + 1] - __uint_as_float(h1 << 16)) << 16);
            }
            bhi[nt][c] = as_bf16x8(hw);
            blo[nt][c] = as_bf16x8(lw);
        }
    }

    // this thread's share of a block: tokens (tid >> s) + k*(256 >> s), 16-B chunk tid & mask
    constexpr int CH = DIDX / 8;                  // 16-B chunks per token
    const int ld_tok = tid / CH, ld_dim = (tid % CH) * 8;
    constexpr int TOK_STEP = 256 / CH;
    const int64_t gofs = (int64_t)g * kgs;

    int done_upto = 0;  // runs are found in row order
    for (;;) {
        if (tid == 0) {
            // the run's request, its block range, and the blocks [full_lo,
            // full_hi) that every row of the tile scores with all 128 tokens
            // visible (the common case: no mask needed there)
            int req = -1, blo_ = 0x7fffffff, bhi_ = -1, n_in = 0;
            int full_lo = 0, full_hi = 0x7fffffff;
            for (int i = 0; i < nrows; ++i) {
                if (s_req[i] < 0) continue;   // already served
                if (req < 0) req = s_req[i];
                if (s_req[i] == req) {
                    blo_ = min(blo_, s_slo[i]);
                    bhi_ = max(bhi_, s_pos[i] / kBlk);
                    full_lo = max(full_lo, s_slo[i]);
                    full_hi = min(full_hi, (s_pos[i] + 1) / kBlk);  // blocks < this are whole
                    ++n_in;
                }
            }
            s_run[0] = req;
            s_run[1] = blo_;
            s_run[2] = bhi_;
            s_run[3] = (n_in == kTileRows) ? full_lo : 0;
            s_run[4] = (n_in == kTileRows) ? full_hi : 0;
        }
        __syncthreads();
        const int req = s_run[0], b_first = s_run[1], b_last = s_run[2];
        const int full_lo = s_run[3], full_hi = s_run[4];
        if (req < 0) break;
        (void)done_upto;
        const int32_t *bt = block_table + (int64_t)req * bt_stride;

        // per-lane row state for the two N tiles
        int lim_base[2], slo_r[2], own_r[2];
        bool act[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int i = 32 * w + 16 * nt + (lane & 15);
            act[nt] = s_req[i] == req;
            lim_base[nt] = s_pos[i];
            slo_r[nt] = s_slo[i];
            own_r[nt] = s_pos[i] / kBlk;
        }

        // stage the first block
        u32x4 pre[LD_PER_THREAD];
        {
            const bf16_t *pg = kbase + (int64_t)bt[b_first] * kps + gofs;
#pragma unroll
            for (int k = 0; k < LD_PER_THREAD; ++k)
                pre[k] = ld16(pg + (int64_t)(ld_tok + k * TOK_STEP) * kts + ld_dim);
#pragma unroll
            for (int k = 0; k < LD_PER_THREAD; ++k)
                *reinterpret_cast<u32x4 *>(&kbuf[0][(ld_tok + k * TOK_STEP) * KST + ld_dim]) = pre[k];
        }
        int next_page = (b_first + 1 <= b_last) ? bt[b_first + 1] : 0;
        __syncthreads();

        for (int b = b_first; b <= b_last; ++b) {
            const int cur = (b - b_first) & 1;
            const bool more = b + 1 <= b_last;
            if (more) {
                const bf16_t *pg = kbase + (int64_t)next_page * kps + gofs;
#pragma unroll
                for (int k = 0; k < LD_PER_THREAD; ++k)
                    pre[k] = ld16(pg + (int64_t)(ld_tok + k * TOK_STEP) * kts + ld_dim);
                if (b + 2 <= b_last) next_page = bt[b + 2];
            }
            // per row: tokens t <= lim visible; -1 = row not scored at this block
            int lim[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                lim[nt] = (act[nt] && b >= slo_r[nt] && b <= own_r[nt]) ? lim_base[nt] - b * kBlk
                                                                        : -1;
            float best[2] = {-INFINITY, -INFINITY};
            const bf16_t *kb = &kbuf[cur][0];
            // raised issue priority while this wave feeds the matrix cores, so
            // that a wave with MFMAs ready goes ahead of one in its staging or
            // barrier phase (2-3 % on the 8K prefill chunk)
            __builtin_amdgcn_s_setprio(1);
            if (b >= full_lo && b < full_hi) {
                // every row sees the whole block: plain maxima
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    bf16x8 a[NC];
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        a[c] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
                            kb + (16 * mt + (lane & 15)) * KST + 32 * c + kq));
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            d = mfma16(a[c], bhi[nt][c], d);
                            d = mfma16(a[c], blo[nt][c], d);
                        }
                        best[nt] = fmaxf(best[nt], fmaxf(fmaxf(d[0], d[1]), fmaxf(d[2], d[3])));
                    }
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    bf16x8 a[NC];
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        a[c] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
                            kb + (16 * mt + (lane & 15)) * KST + 32 * c + kq));
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) {
                        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int c = 0; c < NC; ++c) {
                            d = mfma16(a[c], bhi[nt][c], d);
                            d = mfma16(a[c], blo[nt][c], d);
                        }
                        const int t0 = 16 * mt + (lane >> 4) * 4;
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii)
                            best[nt] = fmaxf(best[nt], (t0 + ii <= lim[nt]) ? d[ii] : -INFINITY);
                    }
                }
            }
            __builtin_amdgcn_s_setprio(0);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                float m = wave_max_xor(best[nt], 16);
                m = wave_max_xor(m, 32);
                if (lane < 16 && lim[nt] >= 0) {
                    const int i = 32 * w + 16 * nt + lane;
                    scores[((int64_t)(row0 + i) * G + g) * score_stride + b] = m * scale;
                }
            }
            if (more) {
#pragma unroll
                for (int k = 0; k < LD_PER_THREAD; ++k)
                    *reinterpret_cast<u32x4 *>(
                        &kbuf[cur ^ 1][(ld_tok + k * TOK_STEP) * KST + ld_dim]) = pre[k];
            }
            __syncthreads();
        }
        // mark this run's rows served
        if (tid < kTileRows && s_req[tid] == req) s_req[tid] = -1;
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_index_score_tiled(const msa_dims_t &d, int rows, const bf16_t *q_idx,
                                    const msa_view_t &kv, const int32_t *block_table,
                                    int bt_stride, const int32_t *row_req, const int32_t *row_pos,
                                    const int32_t *blk_lo, float *scores, int score_stride,
                                    hipStream_t stream) {
    const float scale = 1.0f / sqrtf((float)d.d_idx);
    const bf16_t *kb = static_cast<const bf16_t *>(kv.base);
    const int64_t tiles = (rows + kTileRows - 1) / kTileRows;
    const dim3 grid((unsigned)(tiles * d.G)), block(256);
    if (d.d_idx == 128)
        hipLaunchKernelGGL(index_score_tiled_kernel<128>, grid, block, 0, stream, rows, d.G,
                           d.n_idx, q_idx, kb, kv.page_stride, kv.group_stride, kv.token_stride,
                           block_table, bt_stride, row_req, row_pos, blk_lo, scores, score_stride,
                           scale);
    else
        hipLaunchKernelGGL(index_score_tiled_kernel<64>, grid, block, 0, stream, rows, d.G,
                           d.n_idx, q_idx, kb, kv.page_stride, kv.group_stride, kv.token_stride,
                           block_table, bt_stride, row_req, row_pos, blk_lo, scores, score_stride,
                           scale);
    return hipGetLastError();
}

}  // namespace msa

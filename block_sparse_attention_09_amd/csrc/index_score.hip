// index_score.hip -- block scores of the MSA indexer (gfx950).
//
// Pages: decode index-scoring section (解码索引评分内核优化) of "Together AI 解析如何
// 高效服务 MiniMax M3": the scan compares the query-side index vectors with every
// candidate key-side index vector, reduces each 128-token block to one score and
// sits on the critical path of every generated token; its cost grows with the
// context.  The pages' own kernel puts the 128-token key block on the MMA M
// dimension and the few query vectors, padded, on N.
//
// Score of block b for (row, group):  max over visible tokens t of
//     sum_j q_j . k_t / sqrt(d_idx)
// computed here as qbar . k_t with qbar = sum_j q_j formed in fp32 and split
// into bf16 hi + lo halves (hi = bf16(qbar), lo = bf16(qbar - hi)), so two bf16
// MFMA passes give qbar . k with a relative error near 2^-17 per term against
// the exact sum, accumulated in fp32.  Max commutes with the positive scale,
// which is applied once per block.
//
// Streaming kernel (decode shape: every row reads its own pages).  A wave owns a
// chunk of consecutive blocks of one (row, group) and walks it half a block
// (64 tokens) per step with the next step's loads in flight while the current
// one runs on the matrix cores.  Each lane loads 16 contiguous bytes straight
// into the MFMA A operand (token = M index, 32 dims = K), so the key index goes
// HBM -> VGPR with no LDS round trip; B holds qbar hi/lo in column 0 only.
#include "msa_internal.h"

#include <algorithm>
#include <atomic>

namespace msa {

namespace {

#ifndef MSA_SCORE_NT
#define MSA_SCORE_NT 1
#endif

constexpr int kTilesPerStep = 4;   // 4 x 16 tokens = half a block per register buffer
constexpr int kMaxChunk = 64;      // chunk length bound: one page id per lane

template <int DIDX>
struct StepBuf {
    bf16x8 a[kTilesPerStep][DIDX / 32];
};

// Key-index stream: read once, never reused -> non-temporal loads.
__device__ __forceinline__ u32x4 ld16_stream(const bf16_t *p) {
#if MSA_SCORE_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#else
    return ld16(p);
#endif
}

template <int DIDX>
__device__ __forceinline__ void load_step(StepBuf<DIDX> &buf, const bf16_t *page_base, int64_t kts,
                                          int half, int lane) {
    const int kq = (lane >> 4) * 8;
#pragma unroll
    for (int ti = 0; ti < kTilesPerStep; ++ti) {
        const int tok = (half * kTilesPerStep + ti) * 16 + (lane & 15);
        const bf16_t *p = page_base + (int64_t)tok * kts + kq;
#pragma unroll
        for (int c = 0; c < DIDX / 32; ++c) buf.a[ti][c] = as_bf16x8(ld16_stream(p + 32 * c));
    }
}

// Max over the 64 tokens of one half block of qbar . k_t (fp32), tokens after
// pos masked.  tok_base is the position of this lane's first accumulator row.
template <int DIDX>
__device__ __forceinline__ float block_half_max(const StepBuf<DIDX> &buf, const bf16x8 *bhi,
                                                const bf16x8 *blo, int tok_base, int pos) {
    float best = -INFINITY;
#pragma unroll
    for (int ti = 0; ti < kTilesPerStep; ++ti) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DIDX / 32; ++c) {
            d = mfma16(buf.a[ti][c], bhi[c], d);
            d = mfma16(buf.a[ti][c], blo[c], d);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            best = fmaxf(best, (tok_base + ti * 16 + i <= pos) ? d[i] : -INFINITY);
    }
    return best;
}

// Scored range of pair p = (row r, group g): blocks [slo, own], clamped to the
// score row so that no index leaves the caller's buffers.
struct PairInfo {
    int r, g, req, pos, slo, n;  // n = own - slo + 1 scored blocks
};

__device__ __forceinline__ PairInfo pair_info(int p, int G, const int32_t *__restrict__ row_req,
                                              const int32_t *__restrict__ row_pos,
                                              const int32_t *__restrict__ blk_lo, int score_stride) {
    PairInfo pi;
    pi.r = p / G;
    pi.g = p - pi.r * G;
    pi.req = row_req ? row_req[pi.r] : pi.r;
    pi.pos = row_pos[pi.r];
    const int own = min(pi.pos / kBlk, score_stride - 1);
    const int lo = blk_lo ? blk_lo[(int64_t)pi.req * G + pi.g] : 0;
    pi.slo = max(0, lo < own ? lo : own);
    pi.n = max(0, own - pi.slo + 1);
    return pi;
}

// Scores of blocks [b_beg, b_end) of one (row, group), all inside its scored
// range; at most kMaxChunk blocks (their pages are held one per lane).
template <int DIDX>
__device__ __forceinline__ void score_segment(const PairInfo &pi, int b_beg, int b_end, int n_idx,
                                              int G, const bf16_t *__restrict__ q_idx,
                                              const bf16_t *__restrict__ kbase, int64_t kps,
                                              int64_t kgs, int64_t kts,
                                              const int32_t *__restrict__ block_table,
                                              int bt_stride, float *__restrict__ out, float scale,
                                              int lane) {
    const int32_t *bt = block_table + (int64_t)pi.req * bt_stride;
    // the pages of the first (up to 64) blocks and the query index vectors in
    // one round trip
    const int my_page = (lane < b_end - b_beg) ? bt[b_beg + lane] : 0;
    const int kq = (lane >> 4) * 8;
    const bool col0 = (lane & 15) == 0;
    const bf16_t *qb = q_idx + ((int64_t)pi.r * G + pi.g) * n_idx * DIDX + kq;
    float acc[DIDX / 32][8];
#pragma unroll
    for (int c = 0; c < DIDX / 32; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;
    for (int j0 = 0; j0 < n_idx; j0 += 4) {
        u32x4 w[4][DIDX / 32];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int c = 0; c < DIDX / 32; ++c)
                w[jj][c] = (j0 + jj < n_idx) ? ld16(qb + (j0 + jj) * DIDX + 32 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
            for (int c = 0; c < DIDX / 32; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[c][2 * e] += bf16_lo(w[jj][c][e]);
                    acc[c][2 * e + 1] += bf16_hi(w[jj][c][e]);
                }
    }
    // qbar in fp32 -> bf16 hi + lo, placed in B column 0 (lanes 0, 16, 32, 48).
    bf16x8 bhi[DIDX / 32], blo[DIDX / 32];
#pragma unroll
    for (int c = 0; c < DIDX / 32; ++c) {
        u32x4 hw, lw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t h0 = f32_to_bf16_rne(acc[c][2 * e]);
            const uint32_t h1 = f32_to_bf16_rne(acc[c][2 * e + 1]);
            const uint32_t l0 = f32_to_bf16_rne(acc[c][2 * e] - __uint_as_float(h0 << 16));
            const uint32_t l1 = f32_to_bf16_rne(acc[c][2 * e + 1] - __uint_as_float(h1 << 16));
            hw[e] = col0 ? (h0 | (h1 << 16)) : 0u;
            lw[e] = col0 ? (l0 | (l1 << 16)) : 0u;
        }
        bhi[c] = as_bf16x8(hw);
        blo[c] = as_bf16x8(lw);
    }

    const int64_t gofs = (int64_t)pi.g * kgs;
    const int nblk = b_end - b_beg;
    // Two register buffers, one per half block (static indices: no scratch).
    // The loads of the next half (or of the next block's page) are issued
    // before the matrix-core work on the current half.
    StepBuf<DIDX> bufA, bufB;
    const bf16_t *page = kbase + (int64_t)__builtin_amdgcn_readlane(my_page, 0) * kps + gofs;
    load_step<DIDX>(bufA, page, kts, 0, lane);
    for (int bi = 0; bi < nblk; ++bi) {
        const int tok_base = (b_beg + bi) * kBlk + (lane >> 4) * 4;
        load_step<DIDX>(bufB, page, kts, 1, lane);
        float best = block_half_max<DIDX>(bufA, bhi, blo, tok_base, pi.pos);
        if (bi + 1 < nblk) {
            page = kbase + (int64_t)__builtin_amdgcn_readlane(my_page, bi + 1) * kps + gofs;
            load_step<DIDX>(bufA, page, kts, 0, lane);
        }
        best = fmaxf(best, block_half_max<DIDX>(bufB, bhi, blo, tok_base + 64, pi.pos));
        // column 0 of the accumulators lives in lanes 0, 16, 32, 48
        best = wave_max_xor(best, 16);
        best = wave_max_xor(best, 32);
        if (lane == 0) out[b_beg + bi] = best * scale;
    }
}

// Balanced streaming: the scored blocks of all (row, group) pairs, in pair
// order, are cut into nwaves equal slices, one per wave, so a ragged batch
// ends with every wave finishing together instead of a tail of long rows.
// Each wave first sums the pairs' block counts, then walks the pairs again
// with a running prefix and scores the segments that fall in its slice.
// Blocks outside a pair's scored range get -inf from wave p % nwaves.  With
// up to 64 pairs everything the stream needs arrives in one round trip.
template <int DIDX>
__global__ __launch_bounds__(256, 2) void index_score_stream_kernel(
    int rows, int G, int n_idx, const bf16_t *__restrict__ q_idx, const bf16_t *__restrict__ kbase,
    int64_t kps, int64_t kgs, int64_t kts, const int32_t *__restrict__ block_table, int bt_stride,
    const int32_t *__restrict__ row_req, const int32_t *__restrict__ row_pos,
    const int32_t *__restrict__ blk_lo, float *__restrict__ scores, int score_stride, int nwaves,
    float scale) {
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= nwaves) return;  // wave-uniform
    const int pairs = rows * G;

    // The first 64 pairs' metadata is kept from the counting pass, so a batch
    // of up to 64 pairs costs one round trip before the stream starts.
    // Pair w's range (for its -inf fill) is picked up on the way as well.
    int64_t total = 0;
    PairInfo first = {0, 0, 0, 0, 0, 0};
    int fill_slo = 0, fill_n = 0;
    for (int p0 = 0; p0 < pairs; p0 += kWave) {
        const int p = p0 + lane;
        PairInfo pi = {0, 0, 0, 0, 0, 0};
        if (p < pairs) pi = pair_info(p, G, row_req, row_pos, blk_lo, score_stride);
        if (p0 == 0) first = pi;
        if (p0 == (w & ~(kWave - 1))) {
            fill_slo = __shfl(pi.slo, w & (kWave - 1), kWave);
            fill_n = __shfl(pi.n, w & (kWave - 1), kWave);
        }
        int n = pi.n;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m, kWave);
        total += n;
    }
    // -inf for the blocks outside the scored ranges of pairs w, w + nwaves, ...
    for (int p = w; p < pairs; p += nwaves) {
        if (p != w) {
            const PairInfo pi = pair_info(p, G, row_req, row_pos, blk_lo, score_stride);
            fill_slo = pi.slo;
            fill_n = pi.n;
        }
        float *out = scores + (int64_t)p * score_stride;
        for (int b = lane; b < score_stride; b += kWave)
            if (b < fill_slo || b >= fill_slo + fill_n) out[b] = -INFINITY;
    }
    const int64_t beg = total * w / nwaves, end = total * (w + 1) / nwaves;
    if (beg >= end) return;

    int64_t base = 0;  // blocks of the pairs before this batch of 64
    for (int p0 = 0; p0 < pairs && base < end; p0 += kWave) {
        const int p = p0 + lane;
        PairInfo pi = first;
        if (p0 != 0) {
            pi = PairInfo{0, 0, 0, 0, 0, 0};
            if (p < pairs) pi = pair_info(p, G, row_req, row_pos, blk_lo, score_stride);
        }
        int incl = pi.n;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int v = __shfl_up(incl, off, kWave);
            incl += (lane >= off) ? v : 0;
        }
        const int64_t start = base + incl - pi.n;
        uint64_t hits = __ballot(pi.n > 0 && start < end && start + pi.n > beg);
        while (hits) {
            const int l = __builtin_ctzll(hits);
            hits &= hits - 1;
            PairInfo q;
            q.r = __shfl(pi.r, l, kWave);
            q.g = __shfl(pi.g, l, kWave);
            q.req = __shfl(pi.req, l, kWave);
            q.pos = __shfl(pi.pos, l, kWave);
            q.slo = __shfl(pi.slo, l, kWave);
            q.n = __shfl(pi.n, l, kWave);
            const int64_t st = base + __shfl(incl, l, kWave) - q.n;
            const int b_beg = q.slo + (int)max((int64_t)0, beg - st);
            const int b_end = q.slo + (int)min((int64_t)q.n, end - st);
            for (int c0 = b_beg; c0 < b_end; c0 += kMaxChunk)
                score_segment<DIDX>(q, c0, min(c0 + kMaxChunk, b_end), n_idx, G, q_idx, kbase, kps,
                                    kgs, kts, block_table, bt_stride,
                                    scores + ((int64_t)q.r * G + q.g) * score_stride, scale, lane);
        }
        base += __shfl(incl, kWave - 1, kWave);
    }
}

// ---------------------------------------------------------------------------
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
    constexpr int KST = DIDX + 8;      // LDS row stride of a staged block (16-B pad)
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

hipError_t launch_index_score(const msa_dims_t &d, int rows, const bf16_t *q_idx,
                              const msa_view_t &kv, const int32_t *block_table, int bt_stride,
                              const int32_t *row_req, const int32_t *row_pos,
                              const int32_t *blk_lo, int num_reqs, float *scores,
                              int score_stride, hipStream_t stream) {
    const float scale = 1.0f / sqrtf((float)d.d_idx);
    const bf16_t *kb = static_cast<const bf16_t *>(kv.base);
    // Many rows per request (prefill chunks): the tiled kernel shares each key
    // block across 128 rows.  Otherwise every row streams its own pages.
    if ((int64_t)rows >= 64 * (int64_t)num_reqs) {
        const int64_t tiles = (rows + kTileRows - 1) / kTileRows;
        const dim3 grid((unsigned)(tiles * d.G)), block(256);
        if (d.d_idx == 128)
            hipLaunchKernelGGL(index_score_tiled_kernel<128>, grid, block, 0, stream, rows, d.G,
                               d.n_idx, q_idx, kb, kv.page_stride, kv.group_stride,
                               kv.token_stride, block_table, bt_stride, row_req, row_pos, blk_lo,
                               scores, score_stride, scale);
        else
            hipLaunchKernelGGL(index_score_tiled_kernel<64>, grid, block, 0, stream, rows, d.G,
                               d.n_idx, q_idx, kb, kv.page_stride, kv.group_stride,
                               kv.token_stride, block_table, bt_stride, row_req, row_pos, blk_lo,
                               scores, score_stride, scale);
        return hipGetLastError();
    }
    // One wave per resident wave slot of the device (the balanced kernel is
    // meant to run in a single round), but no more than one per 4 blocks.
    static std::atomic<int> resident_waves[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) dev = 0;
    if (resident_waves[dev].load(std::memory_order_relaxed) == 0) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = d.d_idx == 128
                ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, index_score_stream_kernel<128>, 256, 0)
                : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, index_score_stream_kernel<64>, 256, 0);
        if (e != hipSuccess) return e;
        resident_waves[dev].store((cus > 0 && per_cu > 0) ? cus * per_cu * 4 : 4096,
                                  std::memory_order_relaxed);
    }
    const int64_t pairs = (int64_t)rows * d.G;
    const int64_t ub = pairs * score_stride;  // scored blocks, upper bound
    const int nwaves = (int)std::max<int64_t>(
        1, std::min<int64_t>(resident_waves[dev].load(std::memory_order_relaxed), (ub + 3) / 4));
    const dim3 grid((unsigned)((nwaves + 3) / 4)), block(256);
    if (d.d_idx == 128)
        hipLaunchKernelGGL(index_score_stream_kernel<128>, grid, block, 0, stream, rows, d.G,
                           d.n_idx, q_idx, kb, kv.page_stride, kv.group_stride, kv.token_stride,
                           block_table, bt_stride, row_req, row_pos, blk_lo, scores, score_stride,
                           nwaves, scale);
    else
        hipLaunchKernelGGL(index_score_stream_kernel<64>, grid, block, 0, stream, rows, d.G,
                           d.n_idx, q_idx, kb, kv.page_stride, kv.group_stride, kv.token_stride,
                           block_table, bt_stride, row_req, row_pos, blk_lo, scores, score_stride,
                           nwaves, scale);
    return hipGetLastError();
}

}  // namespace msa

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
// Streaming kernel (decode shape: every row reads its own pages).  Each wave
// takes an equal slice of the scored blocks of all (row, group) pairs and
// walks its segments half a block (64 tokens) per step with the next step's
// loads in flight while the current one runs on the matrix cores.  Each lane
// loads 16 contiguous bytes straight into the MFMA A operand (token = M index,
// 32 dims = K), so the key index goes HBM -> VGPR with no LDS round trip; B
// holds qbar hi/lo in column 0 only.  The prefill shape (many rows of one
// request) uses the row-tiled kernel in index_score_tiled.hip instead.
#include "msa_internal.h"

#include <algorithm>
#include <atomic>

namespace msa {

namespace {

constexpr int kTilesPerStep = 4;   // 4 x 16 tokens = half a block per register buffer
constexpr int kMaxChunk = 64;      // chunk length bound: one page id per lane

template <int DIDX>
struct StepBuf {
    bf16x8 a[kTilesPerStep][DIDX / 32];
};

// Key-index stream: read once, never reused -> non-temporal loads.
__device__ __forceinline__ u32x4 ld16_stream(const bf16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
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
    if ((int64_t)rows >= 64 * (int64_t)num_reqs)
        return launch_index_score_tiled(d, rows, q_idx, kv, block_table, bt_stride, row_req,
                                        row_pos, blk_lo, scores, score_stride, stream);
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

// index_score_dev.h -- device pieces of the streaming index scan, shared by
// the streaming scorer (index_score.hip) and the fused small-batch decode step
// (decode_fused.hip), so that both compute every block score with the same
// arithmetic, bit for bit.
//
// Pages: decode index-scoring section (解码索引评分内核优化) of "Together AI 解析如何
// 高效服务 MiniMax M3".  Score of block b for (row, group): max over visible
// tokens t of sum_j q_j . k_t / sqrt(d_idx), computed as qbar . k_t with
// qbar = sum_j q_j formed in fp32 and fp32 fused multiply-adds; the positive
// scale is applied once per block (max commutes with it).
#pragma once

#include <type_traits>

#include "msa_internal.h"

namespace msa {

constexpr int kMaxChunk = 64;      // chunk length bound: one page id per lane

// Half a block (64 tokens) of key index in registers: load j of the wave moves
// 1 KB, tokens 64 h + TPL j + l / CH (TPL = 64 / CH tokens per load), lane l
// holding dims 8 (l % CH) .. + 8 of its token (CH = d_idx / 8 lanes per token
// row), so every load instruction reads whole token rows.
template <int DIDX>
struct StepBuf {
    static constexpr int CH = DIDX / 8;
    static constexpr int TPL = kWave / CH;
    static constexpr int NLD = 64 / TPL;
    u32x4 v[NLD];
};

// Key-index stream: read once, never reused -> non-temporal loads.
__device__ __forceinline__ u32x4 ld16_stream(const bf16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

template <int DIDX>
__device__ __forceinline__ void load_step(StepBuf<DIDX> &buf, const bf16_t *page_base, int64_t kts,
                                          int half, int lane) {
    using B = StepBuf<DIDX>;
    const bf16_t *p = page_base + (int64_t)(64 * half + lane / B::CH) * kts + 8 * (lane % B::CH);
#pragma unroll
    for (int j = 0; j < B::NLD; ++j) buf.v[j] = ld16_stream(p + (int64_t)(B::TPL * j) * kts);
}

// x summed over the CH lanes of a token row, returned in every one of them
// (butterflies over lane partners l ^ 15, l ^ 7, l ^ 2, l ^ 1 within the row,
// each one DPP-fed add; CH = 8 skips the first).
template <int CH>
__device__ __forceinline__ float row_sum(float x) {
    auto dpp_add = [](float v, auto ctrl) {
        return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                              0xf, 0xf, false));
    };
    if constexpr (CH == 16) x = dpp_add(x, std::integral_constant<int, 0x140>{});  // row_mirror
    x = dpp_add(x, std::integral_constant<int, 0x141>{});                          // row_half_mirror
    x = dpp_add(x, std::integral_constant<int, 0x4e>{});                           // quad_perm 2,3,0,1
    x = dpp_add(x, std::integral_constant<int, 0xb1>{});                           // quad_perm 1,0,3,2
    return x;
}

// Max over the 64 tokens of one half block of qbar . k_t (fp32), tokens after
// pos masked.  tok is the position of this lane's token in the first load.
template <int DIDX>
__device__ __forceinline__ float block_half_max(const StepBuf<DIDX> &buf, const float *qv, int tok,
                                                int pos) {
    using B = StepBuf<DIDX>;
    float best = -INFINITY;
#pragma unroll
    for (int j = 0; j < B::NLD; ++j) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s = fmaf(qv[2 * e], bf16_lo(buf.v[j][e]), s);
            s = fmaf(qv[2 * e + 1], bf16_hi(buf.v[j][e]), s);
        }
        s = row_sum<B::CH>(s);
        best = fmaxf(best, (tok + B::TPL * j <= pos) ? s : -INFINITY);
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
// PIPELINED keeps two half blocks in registers (the next one's loads in flight
// while the current one is reduced); without it one half block is loaded and
// reduced at a time, for kernels whose waves have fewer registers (the same
// arithmetic on every block either way).
template <int DIDX, bool PIPELINED = true>
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
    // qbar = sum_j q_j in fp32: this lane's 8 dims, 8 (l % CH) .. + 8
    using B = StepBuf<DIDX>;
    const bf16_t *qb = q_idx + ((int64_t)pi.r * G + pi.g) * n_idx * DIDX + 8 * (lane % B::CH);
    float qv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < n_idx; ++j) {
        const u32x4 w = ld16(qb + j * DIDX);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qv[2 * e] += bf16_lo(w[e]);
            qv[2 * e + 1] += bf16_hi(w[e]);
        }
    }

    const int64_t gofs = (int64_t)pi.g * kgs;
    const int nblk = b_end - b_beg;
    // Two register buffers, one per half block (static indices: no scratch).
    // The loads of the next half (or of the next block's page) are issued
    // before the current half is reduced.
    StepBuf<DIDX> bufA, bufB;
    const bf16_t *page = kbase + (int64_t)__builtin_amdgcn_readlane(my_page, 0) * kps + gofs;
    load_step<DIDX>(bufA, page, kts, 0, lane);
    for (int bi = 0; bi < nblk; ++bi) {
        const int tok = (b_beg + bi) * kBlk + lane / B::CH;
        float best;
        if constexpr (PIPELINED) {
            load_step<DIDX>(bufB, page, kts, 1, lane);
            best = block_half_max<DIDX>(bufA, qv, tok, pi.pos);
            if (bi + 1 < nblk) {
                page = kbase + (int64_t)__builtin_amdgcn_readlane(my_page, bi + 1) * kps + gofs;
                load_step<DIDX>(bufA, page, kts, 0, lane);
            }
            best = fmaxf(best, block_half_max<DIDX>(bufB, qv, tok + 64, pi.pos));
        } else {
            best = block_half_max<DIDX>(bufA, qv, tok, pi.pos);
            load_step<DIDX>(bufA, page, kts, 1, lane);
            best = fmaxf(best, block_half_max<DIDX>(bufA, qv, tok + 64, pi.pos));
            if (bi + 1 < nblk) {
                page = kbase + (int64_t)__builtin_amdgcn_readlane(my_page, bi + 1) * kps + gofs;
                load_step<DIDX>(bufA, page, kts, 0, lane);
            }
        }
        // the token rows of a load are the lane groups of CH lanes
        if (B::CH == 8) best = wave_max_xor(best, 8);
        best = wave_max_xor(best, 16);
        best = wave_max_xor(best, 32);
        if (lane == 0) out[b_beg + bi] = best * scale;
    }
}


// Balanced streaming: the scored blocks of all (row, group) pairs, in pair
// order, are cut into nwaves equal slices, one per wave, so a ragged batch
// ends with every wave finishing together instead of a tail of long rows.
// Wave w first sums the pairs' block counts, then walks the pairs again with a
// running prefix and scores the segments that fall in its slice.  Blocks
// outside a pair's scored range get -inf from wave p % nwaves.  With up to 64
// pairs everything the stream needs arrives in one round trip.  done(p, n) is
// called by the whole wave once this wave's stores for pair p are issued: n = 1
// after its -inf fill of p, n = the number of blocks after its scores of p.
template <int DIDX, class Done>
__device__ __forceinline__ void stream_scan_wave(
    int rows, int G, int n_idx, const bf16_t *__restrict__ q_idx, const bf16_t *__restrict__ kbase,
    int64_t kps, int64_t kgs, int64_t kts, const int32_t *__restrict__ block_table, int bt_stride,
    const int32_t *__restrict__ row_req, const int32_t *__restrict__ row_pos,
    const int32_t *__restrict__ blk_lo, float *__restrict__ scores, int score_stride, int nwaves,
    float scale, int w, int lane, Done &&done) {
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
        done(p, 1);
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
            if (b_end > b_beg) done(q.r * G + q.g, b_end - b_beg);
        }
        base += __shfl(incl, kWave - 1, kWave);
    }
}

}  // namespace msa

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

template <int DIDX>
__global__ __launch_bounds__(256) void index_score_stream_kernel(
    int rows, int G, int n_idx, const bf16_t *__restrict__ q_idx, const bf16_t *__restrict__ kbase,
    int64_t kps, int64_t kgs, int64_t kts, const int32_t *__restrict__ block_table, int bt_stride,
    const int32_t *__restrict__ row_req, const int32_t *__restrict__ row_pos,
    const int32_t *__restrict__ blk_lo, float *__restrict__ scores, int score_stride, int cb,
    int nchunk, float scale) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wave >= (int64_t)rows * G * nchunk) return;  // wave-uniform
    const int chunk = (int)(wave % nchunk);
    const int rg = (int)(wave / nchunk);
    const int g = rg % G;
    const int r = rg / G;
    const int req = row_req ? row_req[r] : r;
    const int pos = row_pos[r];
    const int own = pos / kBlk;
    const int lo = blk_lo ? blk_lo[(int64_t)req * G + g] : 0;
    const int slo = lo < own ? lo : own;  // scored blocks: [slo, own]
    const int b0 = chunk * cb;
    const int b1 = min(b0 + cb, score_stride);
    float *out = scores + ((int64_t)r * G + g) * score_stride;

    // Blocks of the chunk outside the scored range get -inf.
    const int s0 = max(b0, slo);
    const int s1 = min(b1, own + 1);  // scored blocks of this chunk: [s0, s1)
    for (int b = b0 + lane; b < b1; b += kWave)
        if (b < s0 || b >= s1) out[b] = -INFINITY;
    if (s0 >= s1) return;

    // One round trip for everything the chunk needs besides the stream itself:
    // the page of every scored block (one per lane) and the query index vectors.
    const int32_t *bt = block_table + (int64_t)req * bt_stride;
    const int my_page = (lane < s1 - s0) ? bt[s0 + lane] : 0;
    const int kq = (lane >> 4) * 8;
    const bool col0 = (lane & 15) == 0;
    const bf16_t *qb = q_idx + ((int64_t)r * G + g) * n_idx * DIDX + kq;
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

    const int64_t gofs = (int64_t)g * kgs;
    const int nblk = s1 - s0;
    // Two register buffers, one per half block (static indices: no scratch).  The
    // loads of the next half (or of the next block's page) are issued before the
    // matrix-core work on the current half.
    StepBuf<DIDX> bufA, bufB;
    const bf16_t *page = kbase + (int64_t)__builtin_amdgcn_readlane(my_page, 0) * kps + gofs;
    load_step<DIDX>(bufA, page, kts, 0, lane);
    for (int bi = 0; bi < nblk; ++bi) {
        const int tok_base = (s0 + bi) * kBlk + (lane >> 4) * 4;
        load_step<DIDX>(bufB, page, kts, 1, lane);
        float best = block_half_max<DIDX>(bufA, bhi, blo, tok_base, pos);
        if (bi + 1 < nblk) {
            page = kbase + (int64_t)__builtin_amdgcn_readlane(my_page, bi + 1) * kps + gofs;
            load_step<DIDX>(bufA, page, kts, 0, lane);
        }
        best = fmaxf(best, block_half_max<DIDX>(bufB, bhi, blo, tok_base + 64, pos));
        // column 0 of the accumulators lives in lanes 0, 16, 32, 48
        best = wave_max_xor(best, 16);
        best = wave_max_xor(best, 32);
        if (lane == 0) out[s0 + bi] = best * scale;
    }
}

}  // namespace

hipError_t launch_index_score(const msa_dims_t &d, int rows, const bf16_t *q_idx,
                              const msa_view_t &kv, const int32_t *block_table, int bt_stride,
                              const int32_t *row_req, const int32_t *row_pos,
                              const int32_t *blk_lo, int num_reqs, float *scores,
                              int score_stride, hipStream_t stream) {
    (void)num_reqs;
    // Chunk length: enough waves to fill 256 CUs several times over.
    const int64_t pairs = (int64_t)rows * d.G;
#ifndef MSA_SCORE_WAVES_TARGET
#define MSA_SCORE_WAVES_TARGET 4096
#endif
    int cb = (int)((pairs * score_stride) / MSA_SCORE_WAVES_TARGET);
    cb = cb < 2 ? 2 : (cb > 16 ? 16 : cb);
    static_assert(16 <= kMaxChunk, "chunk pages are held one per lane");
    const int nchunk = (score_stride + cb - 1) / cb;
    const int64_t waves = pairs * nchunk;
    const int64_t blocks = (waves + 3) / 4;
    const float scale = 1.0f / sqrtf((float)d.d_idx);
    const bf16_t *kb = static_cast<const bf16_t *>(kv.base);
    if (d.d_idx == 128)
        hipLaunchKernelGGL(index_score_stream_kernel<128>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, rows, d.G, d.n_idx, q_idx, kb, kv.page_stride,
                           kv.group_stride, kv.token_stride, block_table, bt_stride, row_req,
                           row_pos, blk_lo, scores, score_stride, cb, nchunk, scale);
    else
        hipLaunchKernelGGL(index_score_stream_kernel<64>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, rows, d.G, d.n_idx, q_idx, kb, kv.page_stride,
                           kv.group_stride, kv.token_stride, block_table, bt_stride, row_req,
                           row_pos, blk_lo, scores, score_stride, cb, nchunk, scale);
    return hipGetLastError();
}

}  // namespace msa

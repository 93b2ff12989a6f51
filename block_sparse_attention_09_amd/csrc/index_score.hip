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

constexpr int kTilesPerStep = 4;             // 4 x 16 tokens = half a block per step
constexpr int kStepsPerBlock = kBlk / (16 * kTilesPerStep);

template <int DIDX>
struct StepBuf {
    bf16x8 a[kTilesPerStep][DIDX / 32];
};

template <int DIDX>
__device__ __forceinline__ void load_step(StepBuf<DIDX> &buf, const bf16_t *page_base, int64_t kts,
                                          int half, int lane) {
    const int kq = (lane >> 4) * 8;
#pragma unroll
    for (int ti = 0; ti < kTilesPerStep; ++ti) {
        const int tok = (half * kTilesPerStep + ti) * 16 + (lane & 15);
        const bf16_t *p = page_base + (int64_t)tok * kts + kq;
#pragma unroll
        for (int c = 0; c < DIDX / 32; ++c) buf.a[ti][c] = as_bf16x8(ld16(p + 32 * c));
    }
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

    // qbar = sum_j q_j in fp32, split into bf16 hi/lo, placed in B column 0.
    const int kq = (lane >> 4) * 8;
    const bool col0 = (lane & 15) == 0;
    bf16x8 bhi[DIDX / 32], blo[DIDX / 32];
    const bf16_t *qb = q_idx + ((int64_t)r * G + g) * n_idx * DIDX;
#pragma unroll
    for (int c = 0; c < DIDX / 32; ++c) {
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int j = 0; j < n_idx; ++j) {
            const u32x4 w = ld16(qb + j * DIDX + 32 * c + kq);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += bf16_lo(w[e]);
                acc[2 * e + 1] += bf16_hi(w[e]);
            }
        }
        u32x4 hw, lw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t h0 = f32_to_bf16_rne(acc[2 * e]), h1 = f32_to_bf16_rne(acc[2 * e + 1]);
            uint32_t l0 = f32_to_bf16_rne(acc[2 * e] - __uint_as_float(h0 << 16));
            uint32_t l1 = f32_to_bf16_rne(acc[2 * e + 1] - __uint_as_float(h1 << 16));
            hw[e] = col0 ? (h0 | (h1 << 16)) : 0u;
            lw[e] = col0 ? (l0 | (l1 << 16)) : 0u;
        }
        bhi[c] = as_bf16x8(hw);
        blo[c] = as_bf16x8(lw);
    }

    const int64_t gofs = (int64_t)g * kgs;
    const int32_t *bt = block_table + (int64_t)req * bt_stride;
    const int nsteps = (s1 - s0) * kStepsPerBlock;

    StepBuf<DIDX> buf[2];
    float best = -INFINITY;
    const bf16_t *page_cur = kbase + (int64_t)bt[s0] * kps + gofs;
    load_step<DIDX>(buf[0], page_cur, kts, 0, lane);

    for (int step = 0; step < nsteps; ++step) {
        const int cur = step & 1;
        const int b = s0 + step / kStepsPerBlock;
        const int half = step % kStepsPerBlock;
        // issue the next step's loads (next half, or the next block's page) first
        if (step + 1 < nsteps) {
            const int nb_ = s0 + (step + 1) / kStepsPerBlock;
            const bf16_t *page_next =
                (nb_ == b) ? page_cur : kbase + (int64_t)bt[nb_] * kps + gofs;
            load_step<DIDX>(buf[cur ^ 1], page_next, kts, (step + 1) % kStepsPerBlock, lane);
            if (nb_ != b) page_cur = page_next;
        }
#pragma unroll
        for (int ti = 0; ti < kTilesPerStep; ++ti) {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < DIDX / 32; ++c) {
                d = mfma16(buf[cur].a[ti][c], bhi[c], d);
                d = mfma16(buf[cur].a[ti][c], blo[c], d);
            }
            const int tok0 = b * kBlk + (half * kTilesPerStep + ti) * 16 + (lane >> 4) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) best = fmaxf(best, (tok0 + i <= pos) ? d[i] : -INFINITY);
        }
        if (half == kStepsPerBlock - 1) {
            // column 0 lives in lanes 0, 16, 32, 48
            float m = wave_max_xor(best, 16);
            m = wave_max_xor(m, 32);
            if (lane == 0) out[b] = m * scale;
            best = -INFINITY;
        }
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
    int cb = (int)((pairs * score_stride) / 16384);
    cb = cb < 2 ? 2 : (cb > 16 ? 16 : cb);
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

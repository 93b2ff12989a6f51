// merge.hip -- log-sum-exp reduction of per-block partial outputs (gfx950).
//
// Pages: "Together AI 解析如何高效服务 MiniMax M3", KV 块主序稀疏注意力: every KV
// block yields a partial O, and a final reduction based on log-sum-exp rescales
// the partial outputs and sums them.  (The page's own formula did not survive;
// this is the standard combination.)
//   m = max_s lse_s,  w_s = exp(lse_s - m),
//   o = sum_s w_s o_s / sum_s w_s,   lse = m + ln(sum_s w_s)
// Slots with lse = -inf (empty) are skipped.
//
// HBM-bound: 16 lanes own one (row, head) pair, 8 dims (16 B) each, so a wave
// streams four pairs' partial rows with 16-byte loads.
#include "msa_internal.h"

namespace msa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One wave serves four (row, head) pairs; 16 lanes per pair, 8 dims each.
// Slots go in batches of 8 with all their loads issued together, so a short
// merge (decode: a few hundred pairs) costs a few memory round trips rather
// than one per slot.
constexpr int kBatch = 8;

__global__ __launch_bounds__(64) void lse_merge_kernel(int64_t pairs, int nslot,
                                                       const bf16_t *__restrict__ o_part,
                                                       const float *__restrict__ lse_part,
                                                       bf16_t *__restrict__ o,
                                                       float *__restrict__ lse) {
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    if (pair >= pairs) return;
    const float *ls = lse_part + pair * nslot;
    const bf16_t *op = o_part + pair * nslot * 128 + sub * 8;
    float m = -INFINITY;
    for (int s0 = 0; s0 < nslot; s0 += kBatch) {
        float l[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) l[i] = (s0 + i < nslot) ? ls[s0 + i] : -INFINITY;
#pragma unroll
        for (int i = 0; i < kBatch; ++i) m = fmaxf(m, l[i]);
    }
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float wsum = 0.f;
    if (m != -INFINITY) {
        for (int s0 = 0; s0 < nslot; s0 += kBatch) {
            float l[kBatch];
            u32x4 v[kBatch];
#pragma unroll
            for (int i = 0; i < kBatch; ++i) l[i] = (s0 + i < nslot) ? ls[s0 + i] : -INFINITY;
#pragma unroll
            for (int i = 0; i < kBatch; ++i)  // empty slots (lse = -inf) are never read
                v[i] = (l[i] != -INFINITY) ? ld16(op + (int64_t)(s0 + i) * 128) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const float w = __builtin_amdgcn_exp2f((l[i] - m) * kLog2e);  // 0 for empty
                wsum += w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += w * bf16_lo(v[i][e]);
                    acc[2 * e + 1] += w * bf16_hi(v[i][e]);
                }
            }
        }
    }
    u32x4 out;
    if (m == -INFINITY) {
        out = u32x4{0u, 0u, 0u, 0u};
    } else {
        const float inv = 1.f / wsum;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    }
    *reinterpret_cast<u32x4 *>(o + pair * 128 + sub * 8) = out;
    if (lse && sub == 0)
        lse[pair] = (m == -INFINITY) ? -INFINITY : m + __builtin_amdgcn_logf(wsum) * kLn2;
}

}  // namespace

hipError_t launch_lse_merge(int rows, int H, int nslot, const bf16_t *o_part,
                            const float *lse_part, bf16_t *o, float *lse, hipStream_t stream) {
    const int64_t pairs = (int64_t)rows * H;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)((pairs + 3) / 4)), dim3(64), 0, stream,
                       pairs, nslot, o_part, lse_part, o, lse);
    return hipGetLastError();
}

}  // namespace msa

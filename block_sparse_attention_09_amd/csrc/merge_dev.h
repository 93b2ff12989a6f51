// merge_dev.h -- log-sum-exp combination of one (row, head) pair's slot
// partials by 16 lanes, shared by the merge kernel (merge.hip) and the fused
// small-batch decode step (decode_fused.hip), so that both produce the same
// output bit for bit (gfx950).
//
// Pages: "Together AI 解析如何高效服务 MiniMax M3", KV 块主序稀疏注意力: every KV
// block yields a partial O, and a final reduction based on log-sum-exp rescales
// the partial outputs and sums them:
//   m = max_s lse_s,  w_s = exp(lse_s - m),
//   o = sum_s w_s o_s / sum_s w_s,   lse = m + ln(sum_s w_s)
// Slots with lse = -inf (empty) are skipped.
#pragma once

#include "msa_internal.h"

namespace msa {

// Slots go in batches of kMergeBatch (one batch holds a top-16 + own
// selection) with every load of a batch -- the batch's LSEs and all its partial
// rows -- issued before any is used, so a pair costs one memory round trip per
// batch; batches are combined with a running maximum.  An empty slot (lse =
// -inf) gets weight 0 and its row is excluded by a select, so whatever that row
// holds never reaches the result.  The 16 lanes sub = 0 .. 15 of one aligned
// 16-lane group own pair `pair`, 8 dims (16 B) each; lse may be NULL.
constexpr int kMergeBatch = 17;
static_assert(kMergeBatch == 17, "the LSE hand-round covers 16 lanes plus one");

__device__ __forceinline__ void merge_pair16(int64_t pair, int H, int nslot,
                                             const bf16_t *__restrict__ o_part,
                                             const float *__restrict__ lse_part,
                                             bf16_t *__restrict__ o, float *__restrict__ lse,
                                             int sub) {
    // this pair's LSEs: lse_part [rows][nslot][H], slot s at ls[s * H]
    const int64_t row = pair / H;
    const float *ls = lse_part + row * nslot * H + (pair - row * H);
    const bf16_t *op = o_part + pair * nslot * 128 + sub * 8;
    float m = -INFINITY, wsum = 0.f;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s0 = 0; s0 < nslot; s0 += kMergeBatch) {
        float l[kMergeBatch];
        u32x4 v[kMergeBatch];
        // the batch's LSEs: one load per lane (lane sub holds slot s0 + sub, lane
        // 0 also slot s0 + 16), handed round the 16 lanes of the pair
        const float la = (s0 + sub < nslot)
                             ? __builtin_nontemporal_load(ls + (int64_t)(s0 + sub) * H)
                             : -INFINITY;
        const float lb = (sub == 0 && s0 + 16 < nslot)
                             ? __builtin_nontemporal_load(ls + (int64_t)(s0 + 16) * H)
                             : -INFINITY;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            const bool in = s0 + i < nslot;
            l[i] = (i < 16) ? __shfl(la, i, 16) : __shfl(lb, 0, 16);
            v[i] = in ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                            op + (int64_t)(s0 + i) * 128))
                      : u32x4{0u, 0u, 0u, 0u};
        }
        float mb = m;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) mb = fmaxf(mb, l[i]);
        if (mb == -INFINITY) continue;  // nothing valid yet
        const float rescale = __builtin_amdgcn_exp2f((m - mb) * kLog2e);  // 0 when m = -inf
        wsum *= rescale;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= rescale;
        m = mb;
#pragma unroll
        for (int i = 0; i < kMergeBatch; ++i) {
            const bool use = l[i] != -INFINITY;
            const float w = use ? __builtin_amdgcn_exp2f((l[i] - m) * kLog2e) : 0.f;
            wsum += w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += use ? w * bf16_lo(v[i][e]) : 0.f;
                acc[2 * e + 1] += use ? w * bf16_hi(v[i][e]) : 0.f;
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
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4 *>(o + pair * 128 + sub * 8));
    if (lse && sub == 0)
        lse[pair] = (m == -INFINITY) ? -INFINITY : m + __builtin_amdgcn_logf(wsum) * kLn2;
}

}  // namespace msa

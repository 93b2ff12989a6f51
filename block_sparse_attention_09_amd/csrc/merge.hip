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
// streams four pairs' partial rows with 16-byte loads; the 32 pairs of a
// workgroup are consecutive heads, whose LSEs for one slot are contiguous.  Partials are read once:
// the loads are non-temporal (5 % faster on the prefill shape than cached ones),
// and each LSE is loaded by one lane and shuffled to the others (a further 6 %).
// The output rows are stored non-temporally too: on the prefill shape, right
// after the block-major kernel has written its 2.3 GB of partials, cached
// stores cost 8 % more time than non-temporal ones.
#include "merge_dev.h"
#include "msa_internal.h"

namespace msa {

namespace {

// 16 lanes own one (row, head) pair (merge_pair16); a workgroup of THREADS
// threads serves THREADS / 16 pairs, consecutive heads.  Large merges
// (prefill) take 512 threads, so that the 32 heads' LSEs of one slot fill one
// 128-byte line; small ones (decode) 256, for twice the workgroups.
template <int THREADS>
__global__ __launch_bounds__(THREADS) void lse_merge_kernel(int64_t pairs, int H, int nslot,
                                                                  const bf16_t *__restrict__ o_part,
                                                                  const float *__restrict__ lse_part,
                                                                  bf16_t *__restrict__ o,
                                                                  float *__restrict__ lse) {
    const int64_t pair = (int64_t)blockIdx.x * (THREADS / 16) + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
    if (pair >= pairs) return;  // whole 16-lane groups leave together
    merge_pair16(pair, H, nslot, o_part, lse_part, o, lse, sub);
}

}  // namespace

hipError_t launch_lse_merge(int rows, int H, int nslot, const bf16_t *o_part,
                            const float *lse_part, bf16_t *o, float *lse, hipStream_t stream) {
    const int64_t pairs = (int64_t)rows * H;
    // 512 threads once the merge fills the device several times over
    if (pairs >= (int64_t)1 << 16)
        hipLaunchKernelGGL(lse_merge_kernel<512>, dim3((unsigned)((pairs + 31) / 32)), dim3(512),
                           0, stream, pairs, H, nslot, o_part, lse_part, o, lse);
    else
        hipLaunchKernelGGL(lse_merge_kernel<256>, dim3((unsigned)((pairs + 15) / 16)), dim3(256),
                           0, stream, pairs, H, nslot, o_part, lse_part, o, lse);
    return hipGetLastError();
}

}  // namespace msa

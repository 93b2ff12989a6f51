// decode_fused.hip -- the whole decode step in one launch (gfx950).
//
// Pages ("Together AI 解析如何高效服务 MiniMax M3"): the new smaller kernels of the
// path, the top-k among them, are named as fusion candidates (未来工作); the
// steps fused here are the index scan (解码索引评分内核优化), the top-k selection
// and page-table lookup feeding the paged decode attention (将 MSA 与分页注意力
// 集成), and the log-sum-exp combination of the per-block partials (KV 块主序稀疏
// 注意力).
//
// One grid of 256-thread workgroups does the work of three kernels: each
// workgroup takes a ticket (an atomic counter) when it starts, so tickets
// follow the order in which workgroups actually run.
//   tickets 0 .. nscan - 1     scan: the four waves of ticket t are waves
//                              4t .. 4t + 3 of the balanced streaming scan
//                              (stream_scan_wave, the code of msa_index_score);
//                              after its stores for a pair, a wave publishes how
//                              many of that pair's blocks it scored (or its -inf
//                              fill) with a release fence and an atomic add.
//   the other tickets          one (row, group, slot) unit each: wait until the
//                              pair's count is complete (its scored blocks and
//                              its fill), then select and attend exactly as
//                              msa_sparse_attn_decode_select does (select_unit);
//                              the last unit of a pair to publish its partial
//                              merges the pair (merge_pair16, the code of
//                              msa_lse_merge).
// A unit only ever waits for scan tickets, which were taken before its own by
// workgroups that were already running and never wait themselves, so every
// wait ends; a bound on the number of polls (it raises a flag in the sync
// words) keeps every workgroup finite regardless.  The last unit of a pair
// and the last workgroup overall reset the counters they used, so the sync
// words are zero again when the kernel ends: no clearing launch is needed and
// the step can be captured in a graph.  Every output is bit-identical to
// msa_index_score, msa_sparse_attn_decode_select and msa_lse_merge run one
// after the other.
//
// An agent-scope fence writes back the L2 of the wave's XCD (release) or
// invalidates it (acquire), so the number of waves that fence is kept small:
// the single launch is meant for short, small batches, where three launches
// and the gaps between them, not bytes, set the step time.
#include "decode_dev.h"
#include "index_score_dev.h"
#include "merge_dev.h"
#include "msa_internal.h"

#include <algorithm>
#include <atomic>

namespace msa {

namespace {

__device__ __forceinline__ int load_agent(const int32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int32_t *p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int DIDX, int HG, int KPT>
__global__ __launch_bounds__(kDecThreads, 2) void decode_step_kernel(AttnArgs a, StepArgs f,
                                                                     float scale_log2) {
    __shared__ __attribute__((aligned(16))) char lds[4 * kWaveLds];
    __shared__ int s_ticket, s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int pairs = a.rows * a.G;
    const int nscan = f.nscan_waves / 4;
    const int total = nscan + pairs * a.nslot;
    int32_t *ticket = f.sync, *finished = f.sync + 1, *error = f.sync + 2;
    int32_t *scan_done = f.sync + kStepSyncHead, *unit_done = scan_done + pairs;

    if (tid == 0) s_ticket = atomicAdd(ticket, 1);
    __syncthreads();
    const int t = s_ticket;
    if (t < nscan) {
        stream_scan_wave<DIDX>(a.rows, a.G, f.n_idx, f.q_idx, f.kidx, f.kips, f.kigs, f.kits,
                               f.block_table, f.bt_stride, f.row_req, a.row_pos, f.blk_lo,
                               f.scores, f.score_stride, f.nscan_waves, f.index_scale,
                               4 * t + (tid >> 6), lane, [&](int p, int n) {
                                   if (lane == 0) {
                                       __threadfence();  // release this wave's stores of pair p
                                       atomicAdd(&scan_done[p], n);
                                   }
                               });
    } else {
        const int unit = t - nscan;  // (row, group, slot)
        const int p = unit / a.nslot;
        if (tid == 0) {
            // the pair's scan is complete once its scored blocks and its -inf
            // fill are counted
            const PairInfo pi = pair_info(p, a.G, f.row_req, a.row_pos, f.blk_lo, f.score_stride);
            const int need = pi.n + 1;
            for (int polls = 0; load_agent(&scan_done[p]) < need;) {
                __builtin_amdgcn_s_sleep(2);
                if (++polls >= f.spin_limit) {
                    atomicOr(error, 1);
                    break;
                }
            }
            __threadfence();  // acquire: the scores of every scanning wave
        }
        __syncthreads();
        const SelectArgs sa{f.scores, f.score_stride, f.k, f.row_req, f.block_table, f.bt_stride,
                            f.sel, f.page_table};
        select_unit<HG, KPT>(a, sa, lds, unit, scale_log2);
        __syncthreads();  // this unit's partial is stored
        if (tid == 0) {
            __threadfence();  // release the partial
            s_last = atomicAdd(&unit_done[p], 1) == a.nslot - 1;
            if (s_last) __threadfence();  // acquire the pair's other partials
        }
        __syncthreads();
        if (s_last) {
            if (tid < HG * 16) {
                const int r = p / a.G, g = p - r * a.G, H = a.G * HG;
                merge_pair16((int64_t)r * H + g * HG + (tid >> 4), H, a.nslot, a.o_part,
                             a.lse_part, f.o, f.lse, tid & 15);
            }
            if (tid == 0) {  // every wait and count of this pair is over
                store_agent(&scan_done[p], 0);
                store_agent(&unit_done[p], 0);
            }
        }
    }
    if (tid == 0 && atomicAdd(finished, 1) == total - 1) {
        // every workgroup has taken its ticket and finished: reset for the next call
        store_agent(ticket, 0);
        store_agent(finished, 0);
    }
}

template <int DIDX, int KPT>
void launch_step(const AttnArgs &a, const StepArgs &f, float sl2, dim3 grid, hipStream_t stream) {
    const dim3 block(kDecThreads);
    switch (a.Hg) {
        case 1: hipLaunchKernelGGL((decode_step_kernel<DIDX, 1, KPT>), grid, block, 0, stream, a, f, sl2); break;
        case 2: hipLaunchKernelGGL((decode_step_kernel<DIDX, 2, KPT>), grid, block, 0, stream, a, f, sl2); break;
        case 4: hipLaunchKernelGGL((decode_step_kernel<DIDX, 4, KPT>), grid, block, 0, stream, a, f, sl2); break;
        case 8: hipLaunchKernelGGL((decode_step_kernel<DIDX, 8, KPT>), grid, block, 0, stream, a, f, sl2); break;
        default: hipLaunchKernelGGL((decode_step_kernel<DIDX, 16, KPT>), grid, block, 0, stream, a, f, sl2); break;
    }
}

}  // namespace

bool decode_step_supported(int d_idx, int score_stride) {
    return (d_idx == 64 || d_idx == 128) && score_stride <= kSelectMaxBlocks;
}

hipError_t launch_decode_step(const AttnArgs &a, StepArgs f, int d_idx, hipStream_t stream) {
    if (!decode_step_supported(d_idx, f.score_stride)) return hipErrorInvalidValue;
    // scan waves: one per scored block, at most eight per CU (rounded up to
    // whole workgroups)
    static std::atomic<int> resident_waves[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) dev = 0;
    if (resident_waves[dev].load(std::memory_order_relaxed) == 0) {
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        resident_waves[dev].store(cus > 0 ? cus * 8 : 2048, std::memory_order_relaxed);
    }
    const int64_t pairs = (int64_t)a.rows * a.G;
    const int64_t waves = std::max<int64_t>(
        1, std::min<int64_t>(resident_waves[dev].load(std::memory_order_relaxed),
                             pairs * f.score_stride));
    f.nscan_waves = (int)((waves + 3) / 4 * 4);
    f.spin_limit = 1 << 20;
    const float sl2 = a.sm_scale * kLog2e;
    const dim3 grid((unsigned)(f.nscan_waves / 4 + pairs * a.nslot));
    if (f.score_stride <= 2 * kDecThreads) {
        if (d_idx == 128) launch_step<128, 2>(a, f, sl2, grid, stream);
        else launch_step<64, 2>(a, f, sl2, grid, stream);
    } else {
        if (d_idx == 128) launch_step<128, 4>(a, f, sl2, grid, stream);
        else launch_step<64, 4>(a, f, sl2, grid, stream);
    }
    return hipGetLastError();
}

}  // namespace msa

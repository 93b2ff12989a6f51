// gather.hip -- on-demand copy of the selected KV pages (gfx950).
//
// Pages: future-work section (未来工作) of "Together AI 解析如何高效服务 MiniMax M3":
// the CPU offload of the key index and of the KV cache can be separated, the
// full key index kept loaded and the KV cache loaded on demand from the top-k
// selection.  This copies, for every (row, group, slot) of a page table, the
// K and V tokens of that page and group from a source cache (typically pinned
// host memory) into a compact device pool, one 128-token K/V pair per slot,
// and writes the page table that addresses the pool.
//
// One workgroup per slot; every load instruction of a wave reads four whole
// 256-byte token rows (16 lanes x 16 B per row), the shape that streams best
// over the host link and from HBM, and all of a thread's loads are in flight
// before its first store.
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kRowsPerPass = kGatherThreads / 16;       // token rows per load round
constexpr int kPasses = kBlk / kRowsPerPass;            // rounds per 128-token page

__global__ __launch_bounds__(kGatherThreads) void gather_pages_kernel(
    int64_t units, int G, int nslot, const int32_t *__restrict__ page_table,
    const bf16_t *__restrict__ sk, int64_t skps, int64_t skgs, int64_t skts,
    const bf16_t *__restrict__ sv, int64_t svps, int64_t svgs, int64_t svts,
    bf16_t *__restrict__ dk, bf16_t *__restrict__ dv, int32_t *__restrict__ dst_pt) {
    const int64_t u = blockIdx.x;  // (row * G + g) * nslot + slot
    const int page = page_table[u];
    const int g = (int)((u / nslot) % G);
    if (threadIdx.x == 0) dst_pt[u] = page < 0 ? -1 : (int32_t)u;
    if (page < 0) return;
    const int row = threadIdx.x >> 4, c = (threadIdx.x & 15) * 8;  // token row, dim chunk
    const bf16_t *kp = sk + (int64_t)page * skps + (int64_t)g * skgs + c;
    const bf16_t *vp = sv + (int64_t)page * svps + (int64_t)g * svgs + c;
    u32x4 kx[kPasses], vx[kPasses];
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
        const int t = row + kRowsPerPass * i;
        kx[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(kp + (int64_t)t * skts));
        vx[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(vp + (int64_t)t * svts));
    }
    bf16_t *kd = dk + u * (kBlk * 128) + c;
    bf16_t *vd = dv + u * (kBlk * 128) + c;
#pragma unroll
    for (int i = 0; i < kPasses; ++i) {
        const int t = row + kRowsPerPass * i;
        *reinterpret_cast<u32x4 *>(kd + t * 128) = kx[i];
        *reinterpret_cast<u32x4 *>(vd + t * 128) = vx[i];
    }
}

}  // namespace

hipError_t launch_gather_pages(int rows, int G, int nslot, const int32_t *page_table,
                               const msa_view_t &k, const msa_view_t &v, bf16_t *dst_k,
                               bf16_t *dst_v, int32_t *dst_page_table, hipStream_t stream) {
    const int64_t units = (int64_t)rows * G * nslot;
    hipLaunchKernelGGL(gather_pages_kernel, dim3((unsigned)units), dim3(kGatherThreads), 0, stream,
                       units, G, nslot, page_table, static_cast<const bf16_t *>(k.base),
                       k.page_stride, k.group_stride, k.token_stride,
                       static_cast<const bf16_t *>(v.base), v.page_stride, v.group_stride,
                       v.token_stride, dst_k, dst_v, dst_page_table);
    return hipGetLastError();
}

}  // namespace msa

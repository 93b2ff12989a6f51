// topk.hip -- per (row, KV group) top-k block selection and the page-table
// gather (gfx950).
//
// Pages: the score part of MSA picks the most relevant K blocks for each KV
// group (架构/特性 of "Together AI 解析如何高效服务 MiniMax M3"); each request and
// group has its own top-k boundary (解码索引评分内核优化); decode builds a page
// table from the selected blocks with the KV group folded into the batch
// (将 MSA 与分页注意力集成).
//
// Selection = radix select on order-preserving 32-bit keys of the fp32 scores,
// one workgroup per (row, group): 8-bit digit passes (LDS histogram, one wave
// scans it) find the k-th largest key T and how many keys equal to T are still
// needed.  The passes start at the highest bit where the candidates' keys
// differ and stop as soon as the bucket holding T is taken whole, so a few
// hundred spread scores usually need two passes, not four.  One ordered pass
// then keeps keys above T plus the lowest-index keys equal to it (ties go to
// the lower block index), compared on the bits the passes fixed, and compacts
// them in ascending block order with wave ballots.  The own block is appended last (it is the largest
// index) and the rest is padded with -1.  Integer decisions on the caller's
// fp32 scores only, so the result is exact and deterministic.
#include "msa_internal.h"
#include "topk_select.h"

namespace msa {

namespace {

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;

// Optional page-table output written next to the selection: page of slot i =
// block_table[request][sel[i]], -1 for an empty slot.  With pt == nullptr the
// top-k kernels write the selection only.
struct PageRow {
    const int32_t *bt;  // this row's block-table row
    int32_t *pt;        // this (row, group)'s page-table slots, or nullptr
    __device__ __forceinline__ void put(int i, int b) const {
        if (pt) pt[i] = (b < 0) ? -1 : bt[b];
    }
};
struct PageOut {
    const int32_t *block_table;
    int bt_stride;
    const int32_t *row_req;
    int32_t *pt;
    __device__ __forceinline__ PageRow row(int rg, int G, int k) const {
        PageRow pr{nullptr, nullptr};
        if (pt) {
            const int r = rg / G;
            const int req = row_req ? row_req[r] : r;
            pr.bt = block_table + (int64_t)req * bt_stride;
            pr.pt = pt + (int64_t)rg * (k + 1);
        }
        return pr;
    }
};

// Register-resident variant: one workgroup per (row, group) holds its scores in
// registers (topk_select_regs); THREADS = 64 needs no workgroup barrier beyond
// the single wave's own.
template <int THREADS, int KPT>
__global__ __launch_bounds__(THREADS) void topk_reg_kernel(int G, const float *__restrict__ scores,
                                                           int score_stride,
                                                           const int32_t *__restrict__ row_pos,
                                                           int k, int32_t *__restrict__ sel,
                                                           PageOut po) {
    __shared__ TopkShared<THREADS / kWave> sh;
    const int rg = blockIdx.x;
    const int own = row_pos[rg / G] / kBlk;
    int32_t *out = sel + (int64_t)rg * (k + 1);
    const PageRow pr = po.row(rg, G, k);
    topk_select_regs<THREADS, KPT>(scores + (int64_t)rg * score_stride, score_stride, own, k, sh,
                                   [&](int slot, int b, int) {
                                       out[slot] = b;
                                       pr.put(slot, b);
                                   });
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(int G, const float *__restrict__ scores,
                                                           int score_stride,
                                                           const int32_t *__restrict__ row_pos,
                                                           int k, int32_t *__restrict__ sel,
                                                           PageOut po) {
    __shared__ uint32_t hist[256];
    __shared__ int wave_tot[kTopkWaves];
    __shared__ uint32_t range_xch[2 * kTopkWaves];
    __shared__ int sh_digit, sh_above;

    const int rg = blockIdx.x;
    const int r = rg / G;
    const int tid = threadIdx.x;
    const int own = row_pos[r] / kBlk;
    const float *s = scores + (int64_t)rg * score_stride;
    int32_t *out = sel + (int64_t)rg * (k + 1);
    const PageRow pr = po.row(rg, G, k);

    // number of candidates: blocks before own with a score other than -inf
    int ncand = 0;
    uint32_t klo = ~0u, khi = 0u;
    for (int base = 0; base < own; base += kTopkThreads) {
        const int b = base + tid;
        const float v = (b < own) ? s[b] : -INFINITY;
        const bool valid = v != -INFINITY;
        if (valid) {
            const uint32_t key = order_key(v);
            klo = min(klo, key);
            khi = max(khi, key);
        }
        int t;
        block_excl_count(valid, wave_tot, &t);
        ncand += t;
    }

    uint32_t thresh = 0u, tmask = 0xffffffffu;  // keep keys whose top bits (tmask) > thresh ...
    int take_eq = 0;  // ... plus the first take_eq (in block order) whose top bits == thresh
    if (k == 0) {
        thresh = 0xffffffffu;  // keep nothing but the own block
    } else if (k < ncand) {
        uint32_t lo, hi;
        key_range<kTopkWaves>(klo, khi, range_xch, &lo, &hi);
        uint32_t prefix = 0u, pmask = 0u;
        int remain = k;
        // as in topk_reg_kernel: from the highest differing bit down
        for (int shift = first_shift(lo, hi); shift >= 0; shift = shift > 8 ? shift - 8 : 0) {
            hist[tid] = 0u;
            __syncthreads();
            for (int b = tid; b < own; b += kTopkThreads) {
                const float v = s[b];
                if (v == -INFINITY) continue;
                const uint32_t key = order_key(v);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid < kWave) find_digit(hist, remain, &sh_digit, &sh_above);
            __syncthreads();
            prefix |= (uint32_t)sh_digit << shift;
            pmask |= 255u << shift;
            remain -= sh_above;
            const bool whole_bucket = (int)hist[sh_digit] == remain;
            __syncthreads();
            if (whole_bucket || shift == 0) break;  // selection decided
        }
        thresh = prefix;
        tmask = pmask;
        take_eq = remain;
    }  // else: every candidate is kept (every finite score's key is > 0)

    // ordered pass: keep, compact ascending, append own, pad
    int n_sel = 0, n_eq = 0;
    for (int base = 0; base < own; base += kTopkThreads) {
        const int b = base + tid;
        uint32_t key = 0u;
        bool valid = false;
        if (b < own) {
            const float v = s[b];
            valid = v != -INFINITY;
            key = valid ? order_key(v) : 0u;
        }
        const uint32_t kk = key & tmask;
        const bool is_eq = valid && kk == thresh && take_eq > 0;
        int eq_tot;
        const int eq_rank = n_eq + block_excl_count(is_eq, wave_tot, &eq_tot);
        const bool keep = valid && (kk > thresh || (is_eq && eq_rank < take_eq));
        int keep_tot;
        const int at = n_sel + block_excl_count(keep, wave_tot, &keep_tot);
        if (keep) {
            out[at] = b;
            pr.put(at, b);
        }
        n_sel += keep_tot;
        n_eq += eq_tot;
    }
    for (int i = n_sel + tid; i <= k; i += kTopkThreads) {
        const int b = (i == n_sel) ? own : -1;
        out[i] = b;
        pr.put(i, b);
    }
}

__global__ void page_table_kernel(int64_t n, int G, int nslot, const int32_t *__restrict__ sel,
                                  const int32_t *__restrict__ row_req,
                                  const int32_t *__restrict__ block_table, int bt_stride,
                                  int32_t *__restrict__ pt) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int r = (int)(i / ((int64_t)G * nslot));
    const int req = row_req ? row_req[r] : r;
    const int b = sel[i];
    pt[i] = (b < 0) ? -1 : block_table[(int64_t)req * bt_stride + b];
}

}  // namespace

hipError_t launch_topk(int rows, int G, const float *scores, int score_stride,
                       const int32_t *row_pos, int k, int32_t *sel, hipStream_t stream,
                       const int32_t *row_req, const int32_t *block_table, int bt_stride,
                       int32_t *page_table) {
    const dim3 grid((unsigned)((int64_t)rows * G));
    const PageOut po{block_table, bt_stride, row_req, page_table};
    // scores per (row, group) held in registers: one wave up to 1024 blocks,
    // a 256-thread workgroup up to 16384; beyond that the global-memory kernel
#define MSA_TOPK_REG(T, K)                                                                  \
    hipLaunchKernelGGL((topk_reg_kernel<T, K>), grid, dim3(T), 0, stream, G, scores,        \
                       score_stride, row_pos, k, sel, po)
    // (one wave: as many scores per lane as the row needs, so that no lane
    // converts, counts and ranks empty register slots)
    if (score_stride <= 64 * 8) MSA_TOPK_REG(64, 8);
    else if (score_stride <= 64 * 9) MSA_TOPK_REG(64, 9);
    else if (score_stride <= 64 * 10) MSA_TOPK_REG(64, 10);
    else if (score_stride <= 64 * 12) MSA_TOPK_REG(64, 12);
    else if (score_stride <= 64 * 16) MSA_TOPK_REG(64, 16);
    // longer rows: 1,024 threads, few scores each (2,048 blocks: 14 -> 11 us
    // against 256 threads x 16; 8,192 blocks: 28 -> 20 us against 256 x 32)
    else if (score_stride <= 1024 * 2) MSA_TOPK_REG(1024, 2);
    else if (score_stride <= 1024 * 4) MSA_TOPK_REG(1024, 4);
    else if (score_stride <= 1024 * 8) MSA_TOPK_REG(1024, 8);
    else if (score_stride <= 1024 * 16) MSA_TOPK_REG(1024, 16);
    else hipLaunchKernelGGL(topk_kernel, grid, dim3(kTopkThreads), 0, stream, G, scores,
                            score_stride, row_pos, k, sel, po);
#undef MSA_TOPK_REG
    return hipGetLastError();
}

hipError_t launch_page_table(int rows, int G, const int32_t *sel, int nslot,
                             const int32_t *row_req, const int32_t *block_table, int bt_stride,
                             int32_t *page_table, hipStream_t stream) {
    const int64_t n = (int64_t)rows * G * nslot;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(page_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, n, G,
                       nslot, sel, row_req, block_table, bt_stride, page_table);
    return hipGetLastError();
}

}  // namespace msa

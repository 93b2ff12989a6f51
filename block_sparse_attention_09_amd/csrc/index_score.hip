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
// computed here as qbar . k_t with qbar = sum_j q_j formed in fp32, products
// and sums in fp32 fused multiply-adds (rounding near 2^-24 per operation).
// Max commutes with the positive scale, which is applied once per block.
//
// Streaming kernel (decode shape: every row reads its own pages).  Each wave
// takes an equal slice of the scored blocks of all (row, group) pairs and
// walks its segments half a block (64 tokens) per step with the next step's
// loads in flight while the current one is reduced.  At about one flop per
// byte the scan is bound by HBM, not by arithmetic, so the shape of the loads
// decides its speed: every load instruction of a wave reads whole 256-byte
// token rows (16 lanes x 16 B per row for d_idx 128), which streams at about
// 6.9 TB/s on MI355X, where the 16-token x 64-byte pieces an MFMA operand
// load takes reach about 5.8.  So the dot products run on the vector ALUs
// (eight FMAs per lane per row piece, then a four-step DPP butterfly across
// the row's lanes), which keep up with the stream with room to spare.  The
// prefill shape (many rows of one request share each key block, a dense
// contraction) uses the matrix-core kernel in index_score_tiled.hip instead.
#include "index_score_dev.h"
#include "msa_internal.h"

#include <algorithm>
#include <atomic>

namespace msa {

namespace {

// Balanced streaming (stream_scan_wave): every wave scores an equal slice of
// the scored blocks of all (row, group) pairs.
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
    stream_scan_wave<DIDX>(rows, G, n_idx, q_idx, kbase, kps, kgs, kts, block_table, bt_stride,
                           row_req, row_pos, blk_lo, scores, score_stride, nwaves, scale, w, lane,
                           [](int, int) {});
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
    // meant to run in a single round), but no more than one per block: a small
    // batch (a short context) then has every block's loads in flight at once
    // instead of a few waves walking several blocks one after another.
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
        1, std::min<int64_t>(resident_waves[dev].load(std::memory_order_relaxed), ub));
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

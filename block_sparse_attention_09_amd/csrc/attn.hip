// attn.hip -- sparse attention over the selected KV blocks: decode partials and
// the KV-block-major prefill (gfx950).
//
// Pages ("Together AI 解析如何高效服务 MiniMax M3"):
//  - 架构/特性: the second half of MSA is dense attention of the query tokens
//    over the selected blocks; every head of a KV group shares its selection.
//  - 将 MSA 与分页注意力集成: decode reads the selected blocks through a page
//    table built per (row, KV group).
//  - KV 块主序稀疏注意力: in prefill many queries select the same KV block, so
//    the {query, block} map is inverted into {block, queries}, the block loop is
//    the outer loop and the query loop the inner one, every KV block moves from
//    HBM once, and each block yields partial outputs that a final log-sum-exp
//    reduction rescales and sums.
//
// One workgroup serves one (KV group, page) unit: it stages K (row-major) and V
// (transposed) in LDS once, then its four waves take tiles of 16 query rows
// (16 / Hg query tokens x Hg heads) against the whole 128-token block:
//   S^T = K Q^T    16x16x32 bf16 MFMA, K from LDS, Q straight from global
//   softmax        per query row over the block's causally visible tokens,
//                  exp2 with log2(e) folded into the scale
//   O^T = V^T P^T  16x16x32 bf16 MFMA, P^T repacked in registers to bf16, V^T
//                  from LDS in the permuted token order that matches it
// and writes the normalised partial (bf16) and its natural-log LSE (fp32).
// Decode units hold one query row each; prefill units come from a counting-sort
// inversion of the selection built in the caller's workspace.
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int KST = 136;  // LDS row stride (bf16 elements): 272 B keeps rows off one bank
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnSmem {
    bf16_t k[kBlk * KST];   // K page, [token][dim]
    bf16_t vt[128 * KST];   // V page, [dim][permuted token position]
};

// LDS column of token t in V^T.  Within each 32-token chunk the MFMA K index
// k = 8 b + 4 a + c holds token 16 a + 4 b + c, which is where the S^T
// accumulators of tiles (2 kc, 2 kc + 1) leave P in each lane.
__device__ __forceinline__ int vt_col(int t) {
    return (t & ~31) | (((t >> 2) & 3) << 3) | (((t >> 4) & 1) << 2) | (t & 3);
}

__device__ __forceinline__ bf16x8 lds16(const bf16_t *p) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(p));
}

// Stage one (page, group) of K and V into LDS.  128 tokens x 16 chunks of
// 16 B per tensor; a wave reads 4 whole tokens (1 KB) per load.
__device__ __forceinline__ void stage_kv(AttnSmem &sm, const bf16_t *kp, int64_t kts,
                                         const bf16_t *vp, int64_t vts) {
    const int tid = threadIdx.x;
    u32x4 kw[8], vw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = tid + kAttnThreads * i;
        const int t = c >> 4, d0 = (c & 15) * 8;
        kw[i] = ld16(kp + (int64_t)t * kts + d0);
        vw[i] = ld16(vp + (int64_t)t * vts + d0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = tid + kAttnThreads * i;
        const int t = c >> 4, d0 = (c & 15) * 8;
        *reinterpret_cast<u32x4 *>(&sm.k[t * KST + d0]) = kw[i];
        bf16_t *col = &sm.vt[d0 * KST + vt_col(t)];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            col[(2 * e) * KST] = (bf16_t)(vw[i][e] & 0xffffu);
            col[(2 * e + 1) * KST] = (bf16_t)(vw[i][e] >> 16);
        }
    }
}

// Attention of query tiles tile_begin, tile_begin + tile_step, ... of a unit's
// query list against the block staged in LDS.  Entry e of the list is
// row * nslot + slot.  Every lane owns query row (lane & 15) of the tile.
template <int HG, typename QList>
__device__ __forceinline__ void attend_tiles(const AttnSmem &sm, const AttnArgs &a, int g,
                                             QList qlist, int nq, int tile_begin, int tile_step,
                                             float scale_log2) {
    constexpr int QPT = 16 / HG;  // query tokens per 16-row tile
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, grp = lane >> 4;
    const int H = a.G * HG;
    const int ntiles = (nq + QPT - 1) / QPT;
    for (int tile = tile_begin; tile < ntiles; tile += tile_step) {
        const int qi = tile * QPT + c / HG;
        const bool valid = qi < nq;
        const int entry = qlist(valid ? qi : tile * QPT);
        const int row = entry / a.nslot, slot = entry - row * a.nslot;
        const int h = g * HG + (c % HG);
        const int blk = a.sel[((int64_t)row * a.G + g) * a.nslot + slot];
        const int vis = valid ? (a.row_pos[row] - blk * kBlk) : -1;  // tokens t <= vis

        const bf16_t *qp = a.q + ((int64_t)row * H + h) * 128 + 8 * grp;
        bf16x8 qb[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) qb[c4] = as_bf16x8(ld16(qp + 32 * c4));

        f32x4 s[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
                s[mt] = mfma16(lds16(&sm.k[(16 * mt + c) * KST + 32 * c4 + 8 * grp]), qb[c4], s[mt]);
        }

        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + 4 * grp + i;
                const float z = (t <= vis) ? s[mt][i] * scale_log2 : -INFINITY;
                s[mt][i] = z;
                m = fmaxf(m, z);
            }
        m = wave_max_xor(m, 16);
        m = wave_max_xor(m, 32);
        const float msafe = (m == -INFINITY) ? 0.f : m;
        float l = 0.f;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(s[mt][i] - msafe);
                s[mt][i] = p;
                l += p;
            }
        l = wave_sum_xor(l, 16);
        l = wave_sum_xor(l, 32);

        f32x4 o[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            u32x4 pw;
            pw[0] = pack_bf16x2(s[2 * kc][0], s[2 * kc][1]);
            pw[1] = pack_bf16x2(s[2 * kc][2], s[2 * kc][3]);
            pw[2] = pack_bf16x2(s[2 * kc + 1][0], s[2 * kc + 1][1]);
            pw[3] = pack_bf16x2(s[2 * kc + 1][2], s[2 * kc + 1][3]);
            const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                o[dt] = mfma16(lds16(&sm.vt[(16 * dt + c) * KST + 32 * kc + 8 * grp]), pb, o[dt]);
        }

        if (valid) {
            const float inv = 1.f / l;
            const int64_t oi = ((int64_t)row * H + h) * a.nslot + slot;
            bf16_t *op = a.o_part + oi * 128 + 4 * grp;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                uint2 w;
                w.x = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
                w.y = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
                *reinterpret_cast<uint2 *>(op + 16 * dt) = w;
            }
            if (grp == 0) a.lse_part[oi] = (m + __builtin_amdgcn_logf(l)) * kLn2;
        }
    }
}

// o = 0, lse = -inf for the Hg heads of an empty (row, group, slot).
template <int HG>
__device__ __forceinline__ void write_empty_slot(const AttnArgs &a, int r, int g, int s, int tid,
                                                 int nthreads) {
    const int H = a.G * HG;
    for (int i = tid; i < HG * 16; i += nthreads) {
        const int hh = i >> 4, ch = i & 15;
        const int64_t oi = ((int64_t)r * H + g * HG + hh) * a.nslot + s;
        *reinterpret_cast<u32x4 *>(a.o_part + oi * 128 + ch * 8) = u32x4{0u, 0u, 0u, 0u};
        if (ch == 0) a.lse_part[oi] = -INFINITY;
    }
}

struct SingleEntry {
    int e;
    __device__ int operator()(int) const { return e; }
};

struct ListEntry {
    const int32_t *p;
    __device__ int operator()(int i) const { return p[i]; }
};

// ------------------------------------------------------------------ decode
template <int HG>
__global__ __launch_bounds__(kAttnThreads) void attn_decode_kernel(AttnArgs a, float scale_log2) {
    __shared__ AttnSmem sm;
    const int unit = blockIdx.x;  // (r, g, s)
    const int s = unit % a.nslot;
    const int rg = unit / a.nslot;
    const int g = rg % a.G, r = rg / a.G;
    const int blk = a.sel[unit];
    if (blk < 0) {
        write_empty_slot<HG>(a, r, g, s, threadIdx.x, kAttnThreads);
        return;
    }
    const int64_t page = a.page_table[unit];
    stage_kv(sm, a.k + page * a.kps + (int64_t)g * a.kgs, a.kts,
             a.v + page * a.vps + (int64_t)g * a.vgs, a.vts);
    __syncthreads();
    if ((threadIdx.x >> 6) == 0)
        attend_tiles<HG>(sm, a, g, SingleEntry{r * a.nslot + s}, 1, 0, 1, scale_log2);
}

// ------------------------------------------------------------------ prefill
// Workspace: counts[G*P] | offs[G*P + 1] | list[rows*G*nslot] (int32 each).
__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Count queries per (group, page); empty slots get their zero partials here.
template <int HG>
__global__ void remap_count_kernel(AttnArgs a, int P, int32_t *__restrict__ counts) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (int64_t)a.rows * a.G * a.nslot;
    if (i >= n) return;
    const int s = (int)(i % a.nslot);
    const int rg = (int)(i / a.nslot);
    const int g = rg % a.G, r = rg / a.G;
    if (a.sel[i] < 0) {
        write_empty_slot<HG>(a, r, g, s, 0, 1);
        return;
    }
    atomicAdd(&counts[(int64_t)g * P + a.page_table[i]], 1);
}

// Single-workgroup exclusive scan of counts into offs (n + 1 entries); counts
// is cleared on the way so the scatter can reuse it as a cursor.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void remap_scan_kernel(int32_t *__restrict__ counts,
                                                                  int32_t *__restrict__ offs,
                                                                  int n) {
    __shared__ int wsum[kScanThreads / kWave];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int per = (n + kScanThreads - 1) / kScanThreads;
    const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
    int local = 0;
    for (int i = b0; i < b1; ++i) local += counts[i];
    // inclusive scan inside the wave
    int incl = local;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int v = __shfl_up(incl, off, kWave);
        incl += (lane >= off) ? v : 0;
    }
    if (lane == kWave - 1) wsum[w] = incl;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < w; ++i) before += wsum[i];
    int run = before + incl - local;
    for (int i = b0; i < b1; ++i) {
        const int cnt = counts[i];
        offs[i] = run;
        run += cnt;
        counts[i] = 0;
    }
    if (tid == kScanThreads - 1) offs[n] = before + incl;
}

__global__ void remap_scatter_kernel(AttnArgs a, int P, int32_t *__restrict__ cursor,
                                     const int32_t *__restrict__ offs, int32_t *__restrict__ list) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (int64_t)a.rows * a.G * a.nslot;
    if (i >= n || a.sel[i] < 0) return;
    const int s = (int)(i % a.nslot);
    const int rg = (int)(i / a.nslot);
    const int g = rg % a.G, r = rg / a.G;
    const int64_t u = (int64_t)g * P + a.page_table[i];
    const int at = atomicAdd(&cursor[u], 1);
    list[offs[u] + at] = r * a.nslot + s;
}

template <int HG>
__global__ __launch_bounds__(kAttnThreads) void attn_blockmajor_kernel(
    AttnArgs a, int P, const int32_t *__restrict__ offs, const int32_t *__restrict__ list,
    float scale_log2) {
    __shared__ AttnSmem sm;
    const int64_t u = blockIdx.x;  // (group, page)
    const int o0 = offs[u], nq = offs[u + 1] - o0;
    if (nq == 0) return;
    const int g = (int)(u / P);
    const int64_t page = u % P;
    stage_kv(sm, a.k + page * a.kps + (int64_t)g * a.kgs, a.kts,
             a.v + page * a.vps + (int64_t)g * a.vgs, a.vts);
    __syncthreads();
    attend_tiles<HG>(sm, a, g, ListEntry{list + o0}, nq, threadIdx.x >> 6, kAttnWaves, scale_log2);
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t stream) {
    const float sl2 = a.sm_scale * kLog2e;
    const dim3 grid((unsigned)((int64_t)a.rows * a.G * a.nslot)), block(kAttnThreads);
    switch (a.Hg) {
        case 1: hipLaunchKernelGGL(attn_decode_kernel<1>, grid, block, 0, stream, a, sl2); break;
        case 2: hipLaunchKernelGGL(attn_decode_kernel<2>, grid, block, 0, stream, a, sl2); break;
        case 4: hipLaunchKernelGGL(attn_decode_kernel<4>, grid, block, 0, stream, a, sl2); break;
        case 8: hipLaunchKernelGGL(attn_decode_kernel<8>, grid, block, 0, stream, a, sl2); break;
        default: hipLaunchKernelGGL(attn_decode_kernel<16>, grid, block, 0, stream, a, sl2); break;
    }
    return hipGetLastError();
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t prefill_workspace_bytes(int rows, int G, int nslot, int num_pages) {
    const size_t units = (size_t)G * num_pages;
    return align256(units * 4) + align256((units + 1) * 4) + align256((size_t)rows * G * nslot * 4);
}

hipError_t launch_attn_prefill(const AttnArgs &a, int P, void *workspace, hipStream_t stream) {
    const int64_t units = (int64_t)a.G * P;
    char *ws = static_cast<char *>(workspace);
    int32_t *counts = reinterpret_cast<int32_t *>(ws);
    int32_t *offs = reinterpret_cast<int32_t *>(ws + align256(units * 4));
    int32_t *list = reinterpret_cast<int32_t *>(ws + align256(units * 4) + align256((units + 1) * 4));
    const int64_t n = (int64_t)a.rows * a.G * a.nslot;
    const float sl2 = a.sm_scale * kLog2e;

    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream,
                       counts, units, 0);
    const dim3 eg((unsigned)((n + 255) / 256)), eb(256);
    switch (a.Hg) {
        case 1: hipLaunchKernelGGL(remap_count_kernel<1>, eg, eb, 0, stream, a, P, counts); break;
        case 2: hipLaunchKernelGGL(remap_count_kernel<2>, eg, eb, 0, stream, a, P, counts); break;
        case 4: hipLaunchKernelGGL(remap_count_kernel<4>, eg, eb, 0, stream, a, P, counts); break;
        case 8: hipLaunchKernelGGL(remap_count_kernel<8>, eg, eb, 0, stream, a, P, counts); break;
        default: hipLaunchKernelGGL(remap_count_kernel<16>, eg, eb, 0, stream, a, P, counts); break;
    }
    hipLaunchKernelGGL(remap_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts, offs,
                       (int)units);
    hipLaunchKernelGGL(remap_scatter_kernel, eg, eb, 0, stream, a, P, counts, offs, list);
    const dim3 grid((unsigned)units), block(kAttnThreads);
    switch (a.Hg) {
        case 1: hipLaunchKernelGGL(attn_blockmajor_kernel<1>, grid, block, 0, stream, a, P, offs, list, sl2); break;
        case 2: hipLaunchKernelGGL(attn_blockmajor_kernel<2>, grid, block, 0, stream, a, P, offs, list, sl2); break;
        case 4: hipLaunchKernelGGL(attn_blockmajor_kernel<4>, grid, block, 0, stream, a, P, offs, list, sl2); break;
        case 8: hipLaunchKernelGGL(attn_blockmajor_kernel<8>, grid, block, 0, stream, a, P, offs, list, sl2); break;
        default: hipLaunchKernelGGL(attn_blockmajor_kernel<16>, grid, block, 0, stream, a, P, offs, list, sl2); break;
    }
    return hipGetLastError();
}

}  // namespace msa

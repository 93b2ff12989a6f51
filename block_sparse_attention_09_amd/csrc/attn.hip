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
// Prefill: one workgroup serves one (KV group, page) unit: it stages K
// (row-major) and V (transposed) in LDS once, then its four waves take tiles of
// 32 query rows (32 / Hg query tokens x Hg heads) against the whole 128-token
// block on the 32x32x16 bf16 matrix cores:
//   S^T = K Q^T    K from LDS (A), Q straight from global (B)
//   softmax        per query row over the block's causally visible tokens,
//                  exp2 with log2(e) folded into the scale, fp32 row sums
//   O^T = V^T P^T  V^T from LDS in the token order that matches where the S^T
//                  accumulators leave P, P^T repacked to bf16 in registers
// and writes the normalised partial (bf16) and its natural-log LSE (fp32).
// A workgroup holds 78 KB of LDS, so two workgroups (eight waves) share a CU
// and one wave's softmax overlaps another's matrix-core work.  The units' query
// lists come from a counting-sort inversion of the selection built in the
// caller's workspace.
//
// Decode: one workgroup per (row, group, slot), the block split over its four
// waves (see attn_decode_kernel below).
#include "decode_dev.h"
#include "msa_internal.h"
#include "topk_select.h"

#include <algorithm>
#include <atomic>

namespace msa {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / kWave;
constexpr int KST = 136;  // LDS row stride (bf16 elements): 272 B keeps rows off one bank

// Output stage of a block-major wave: 8 partial rows of 128 dims, padded by
// 16 bytes so that the 8 rows written at once fall in different LDS banks.
constexpr int kStageRow = 128 + 8;

struct AttnSmem {
    bf16_t k[kBlk * KST];   // K page, [token][dim]
    bf16_t vt[128 * KST];   // V page, [dim][permuted token position]
};

// Column order of V^T in LDS: token t sits in column t with bits 2 and 3
// swapped.  In every 16-token PV step the MFMA K index k = 8 h + 4 q + r holds
// token 8 q + 4 h + r of the step, which is where the S^T accumulators leave P
// in lane half h.

__device__ __forceinline__ bf16x8 lds16(const bf16_t *p) {
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(p));
}

// Stage one (page, group) of K and V into LDS.  128 tokens x 16 chunks of
// 16 B per tensor; a wave reads 4 whole tokens (1 KB) per load.  The loads
// are issued first (stage_kv_load) so other work can overlap their latency.
struct KvStage {
    u32x4 kw[8], vw[8];
};

__device__ __forceinline__ void stage_kv_load(KvStage &st, const bf16_t *kp, int64_t kts,
                                              const bf16_t *vp, int64_t vts) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = tid + kAttnThreads * i;
        const int t = c >> 4, d0 = (c & 15) * 8;
        st.kw[i] = ld16(kp + (int64_t)t * kts + d0);
        st.vw[i] = ld16(vp + (int64_t)t * vts + d0);
    }
}

// Writes the staged tiles; K and V rows of tokens past last_tok (seen by no
// query of the unit, possibly never written) are stored as zeros: a zero
// softmax weight times a non-finite V value would still poison P V, and the
// masked scores start from -inf (blockmajor_wave), which a non-finite K row
// would turn into NaN.  V is transposed in LDS: written row-major into the V^T
// area with whole-row 16-byte stores, read back column-wise with the gfx950
// transposing LDS read (each lane of a 16-lane group receives one dimension
// of four consecutive tokens), then written as V^T rows, again 16 bytes per
// lane: no element-wise scatter.  Holds two workgroup barriers.
__device__ __forceinline__ void stage_kv_store(AttnSmem &sm, const KvStage &st, int last_tok) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = tid + kAttnThreads * i;
        const int t = c >> 4, d0 = (c & 15) * 8;
        const u32x4 zero{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(&sm.k[t * KST + d0]) = (t <= last_tok) ? st.kw[i] : zero;
        *reinterpret_cast<u32x4 *>(&sm.vt[t * KST + d0]) = (t <= last_tok) ? st.vw[i] : zero;
    }
    __syncthreads();
    // Piece (dimension block D0 = 16 (pg % 8), column group j = pg / 8) of V^T:
    // rows D0 .. D0 + 15, columns 8 j .. 8 j + 7, which hold tokens T0 .. T0 + 3
    // and T0 + 8 .. T0 + 11 with T0 = 16 (j / 2) + 4 (j % 2) (the column
    // order above: columns 8 j .. 8 j + 3 are tokens T0 .. T0 + 3).  Group c
    // of wave w takes pieces pg = 16 it + 4 w + c; lane s of the group points
    // the transposing read at token T0 + s / 4, dims D0 + 4 (s % 4), and
    // receives dimension D0 + s of the four tokens.
    const int grp = tid >> 4, s16 = tid & 15;
    v4i16 lo[8], hi[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int pg = 16 * it + grp;
        const int D0 = 16 * (pg & 7), j = pg >> 3;
        const int T0 = 16 * (j >> 1) + 4 * (j & 1);
        const bf16_t *src = &sm.vt[(T0 + (s16 >> 2)) * KST + D0 + 4 * (s16 & 3)];
        lo[it] = lds_read_tr(reinterpret_cast<const char *>(src));
        hi[it] = lds_read_tr(reinterpret_cast<const char *>(src + 8 * KST));
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int pg = 16 * it + grp;
        const int D0 = 16 * (pg & 7), j = pg >> 3;
        u32x4 w;
        w[0] = (uint32_t)(uint16_t)lo[it][0] | ((uint32_t)(uint16_t)lo[it][1] << 16);
        w[1] = (uint32_t)(uint16_t)lo[it][2] | ((uint32_t)(uint16_t)lo[it][3] << 16);
        w[2] = (uint32_t)(uint16_t)hi[it][0] | ((uint32_t)(uint16_t)hi[it][1] << 16);
        w[3] = (uint32_t)(uint16_t)hi[it][2] | ((uint32_t)(uint16_t)hi[it][3] << 16);
        *reinterpret_cast<u32x4 *>(&sm.vt[(D0 + s16) * KST + 8 * j]) = w;
    }
}

// Forces the compiler to have x in registers at this point.  Loads and stores
// share one completion counter on this architecture, so once a store is
// outstanding, waiting for any load waits for the store too; the wave therefore
// takes delivery of everything it prefetched just before it issues its stores.
template <typename T>
__device__ __forceinline__ void take_delivery(const T &x) {
    asm volatile("" ::"v"(x));
}

// Per-lane metadata of one query tile (this lane's query row), kept raw so
// that its loads stay in flight until the tile is processed.
struct TileMeta {
    int row, slot, pos, blk;
    bool valid;
};

// One wave's share of a unit: tiles w, w + 4, ... of 32 query rows each.
// Lane l owns query row l % 32 of the tile; lane half h = l / 32 picks which
// tokens (S^T rows) and head dimensions (O^T rows) it holds.
template <int HG>
__device__ __forceinline__ void blockmajor_wave(const AttnSmem &sm, bf16_t *ostage,
                                                const AttnArgs &a, int g,
                                                const int32_t *__restrict__ lst, int nq,
                                                float scale_log2) {
    constexpr int QPT = 32 / HG;  // query tokens per tile
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = lane & 31, h = lane >> 5;
    const int H = a.G * HG;
    const int ntiles = (nq + QPT - 1) / QPT;
    const int my_tiles = ntiles > w ? (ntiles - w + kAttnWaves - 1) / kAttnWaves : 0;
    if (my_tiles == 0) return;
    const int hh = j % HG;

    auto qidx = [&](int t) { return (w + kAttnWaves * t) * QPT + j / HG; };
    auto entry_of = [&](int t) {
        const int qi = qidx(t);
        return lst[(t < my_tiles && qi < nq) ? qi : 0];
    };
    auto load_q = [&](bf16x8 (&qb)[8], int entry) {
        const int row = entry / a.nslot;
        const bf16_t *qp = a.q + ((int64_t)row * H + g * HG + hh) * 128 + 8 * h;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qb[ks] = as_bf16x8(ld16(qp + 16 * ks));
    };
    auto load_meta = [&](int entry, int t) {
        TileMeta m;
        m.row = entry / a.nslot;
        m.slot = entry - m.row * a.nslot;
        m.pos = a.row_pos[m.row];
        m.blk = a.sel[((int64_t)m.row * a.G + g) * a.nslot + m.slot];
        m.valid = t < my_tiles && qidx(t) < nq;
        return m;
    };

    bf16x8 qb[8];
    const int e0 = entry_of(0);
    load_q(qb, e0);
    TileMeta meta = load_meta(e0, 0);
    int ent_next = entry_of(1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) take_delivery(qb[ks]);
    take_delivery(meta.pos);
    take_delivery(meta.blk);
    take_delivery(ent_next);

    for (int t = 0; t < my_tiles; ++t) {
        // K and V^T operands are re-read from LDS for every tile: without this
        // barrier the compiler hoists all 64 fragment reads out of the loop
        // into registers and the wave no longer fits two per SIMD
        asm volatile("" ::: "memory");
        // S^T = K Q^T: four 32-token row tiles, 8 dimension steps of 16.  The
        // causal mask lives in the accumulators' initial values: element 4 q + r
        // of s[mt] (token 32 mt + 8 q + 4 h + r) starts at 0 if the row sees the
        // token and at -inf if not, so the product leaves masked scores at -inf
        // and the softmax below needs no branch (a select after the product would
        // redefine the accumulators and cost a copy of all 64 per tile).  The
        // decision is an integer sign mask: -inf's bits where 32 mt + 8 q + r >
        // vis - 4 h.  K rows no query of the unit sees are zero (stage_kv_store),
        // so every masked product stays -inf.  Tiles whose rows all see the whole
        // block start from zero.
        const int vis = meta.valid ? meta.pos - meta.blk * kBlk : -1;
        f32x16 s[4];
        // the product runs in each branch, so that both define the accumulators
        // from their initial values (zero as the MFMA's inline operand on the
        // common, unmasked path)
        auto qk = [&]() {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    s[mt] = mfma32(lds16(&sm.k[(32 * mt + j) * KST + 16 * ks + 8 * h]), qb[ks],
                                   s[mt]);
        };
        if (__builtin_amdgcn_readfirstlane(__all(vis >= kBlk - 1))) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) s[mt] = f32x16{};
            qk();
        } else {
            const int lim = vis - 4 * h;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int d = lim - (32 * mt + 8 * (e >> 2) + (e & 3));
                    s[mt][e] = __uint_as_float((uint32_t)(d >> 31) & 0xff800000u);
                }
            qk();
        }

        // the next tile's query rows (into the registers just consumed) and metadata
        const bool more = t + 1 < my_tiles;
        TileMeta meta_next = meta;
        if (more) {
            load_q(qb, ent_next);
            meta_next = load_meta(ent_next, t + 1);
            ent_next = entry_of(t + 2);
        }

        // softmax over the block (masked scores are -inf)
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[mt][e]);
        mx = wave_max_xor(mx, 32);
        const float off = (mx == -INFINITY) ? 0.f : -mx * scale_log2;
        float l = 0.f;
        bf16x8 pb[8];  // P^T operand of PV step ks: elements 8 (ks % 2) .. +8 of s[ks / 2]
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][8 * (ks & 1) + e], scale_log2, off));
                l += p[e];
            }
            u32x4 pw;
            pw[0] = pack_bf16x2(p[0], p[1]);
            pw[1] = pack_bf16x2(p[2], p[3]);
            pw[2] = pack_bf16x2(p[4], p[5]);
            pw[3] = pack_bf16x2(p[6], p[7]);
            pb[ks] = as_bf16x8(pw);
        }
        l = wave_sum_xor(l, 32);

        // O^T = V^T P^T: four 32-dim row tiles, 8 token steps of 16
        f32x16 o[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                o[dt] = mfma32(lds16(&sm.vt[(32 * dt + j) * KST + 16 * ks + 8 * h]), pb[ks], o[dt]);

#pragma unroll
        for (int ks = 0; ks < 8; ++ks) take_delivery(qb[ks]);
        take_delivery(meta_next.pos);
        take_delivery(meta_next.blk);
        take_delivery(ent_next);
        // normalised partial: element 4 q + r of o[dt] is dim 32 dt + 8 q + 4 h + r.
        // One lane-half swap per packed pair gives each lane 8 contiguous dims
        // twice per 32-dim tile (lower half: 0..7 and 16..23, upper: 8..15 and
        // 24..31).  The rows then pass through this wave's LDS stage, 8 rows at a
        // time, so that every global store writes 4 whole 256-byte rows: stores
        // that cover a row in 32-byte pieces from 32 rows at once sustain about
        // 3.0 TB/s on random rows, whole rows about 5.0.  The partials (2.3 GB
        // on an 8K-token chunk) far exceed every cache, so they are stored
        // non-temporally: 8 % faster than cached stores, and the merge that
        // reads them back then runs 8 % faster as well.
        {
            const float inv = 1.f / l;
            u32x4 cw[4][2];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                uint32_t pk[4][2];  // [q][pair]: dims 8 q + 4 h + {0,1}, {2,3}
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    pk[q][0] = pack_bf16x2(o[dt][4 * q] * inv, o[dt][4 * q + 1] * inv);
                    pk[q][1] = pack_bf16x2(o[dt][4 * q + 2] * inv, o[dt][4 * q + 3] * inv);
                }
                // A = q 0 and 2 (kept by the lower half), B = q 1 and 3 (kept by the upper)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const auto x = __builtin_amdgcn_permlane32_swap(pk[0][i], pk[1][i], false, false);
                    const auto y = __builtin_amdgcn_permlane32_swap(pk[2][i], pk[3][i], false, false);
                    cw[dt][0][i] = x[0];
                    cw[dt][0][2 + i] = x[1];
                    cw[dt][1][i] = y[0];
                    cw[dt][1][2 + i] = y[1];
                }
            }
            const int64_t oi = ((int64_t)meta.row * H + g * HG + hh) * a.nslot + meta.slot;
            const int oi_lo = (int)(uint32_t)oi, oi_hi = (int)(oi >> 32);
            const int ok = meta.valid ? 1 : 0;
#pragma unroll
            for (int rho = 0; rho < 4; ++rho) {
                if ((j >> 3) == rho) {
                    bf16_t *sr = ostage + (j & 7) * kStageRow + 8 * h;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        *reinterpret_cast<u32x4 *>(sr + 32 * dt) = cw[dt][0];
                        *reinterpret_cast<u32x4 *>(sr + 32 * dt + 16) = cw[dt][1];
                    }
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int rr = 4 * i + (lane >> 4);  // stage row; tile row 8 rho + rr
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(ostage + rr * kStageRow +
                                                                     8 * (lane & 15));
                    const int src = 8 * rho + rr;  // lanes src and src + 32 hold its metadata
                    const int lo = __shfl(oi_lo, src, kWave), hi = __shfl(oi_hi, src, kWave);
                    if (__shfl(ok, src, kWave)) {
                        const int64_t ro = ((int64_t)hi << 32) | (uint32_t)lo;
                        __builtin_nontemporal_store(
                            v, reinterpret_cast<u32x4 *>(a.o_part + ro * 128 + 8 * (lane & 15)));
                    }
                }
            }
            // the Hg heads of a query token: Hg consecutive LSEs (one 32-byte
            // sector for Hg = 8) written by one instruction
            if (meta.valid && h == 0)
                __builtin_nontemporal_store((mx * scale_log2 + __builtin_amdgcn_logf(l)) * kLn2,
                                            a.lse_part + lse_index(a, meta.row, meta.slot,
                                                                   g * HG + hh));
        }
        meta = meta_next;
    }
}

// ------------------------------------------------------------------ prefill
// Workspace: cnt[G*P][W] | counts[G*P] | offs[G*P + 1] | list[rows*G*nslot]
// (int32 each; W = workgroups of the counting sort, cnt unused when W = 0).
// Units are numbered u = page * G + g, so that with the default round-robin
// dispatch over the 8 XCDs the units of one KV group (and its query rows) stay
// on one XCD's L2 when G is 8.
__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Count queries per (page, group); empty slots get their zero partials here.
template <int HG>
__global__ void remap_count_kernel(AttnArgs a, int32_t *__restrict__ counts) {
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
    atomicAdd(&counts[(int64_t)a.page_table[i] * a.G + g], 1);
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

__global__ void remap_scatter_kernel(AttnArgs a, int32_t *__restrict__ cursor,
                                     const int32_t *__restrict__ offs, int32_t *__restrict__ list) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n = (int64_t)a.rows * a.G * a.nslot;
    if (i >= n || a.sel[i] < 0) return;
    const int s = (int)(i % a.nslot);
    const int rg = (int)(i / a.nslot);
    const int g = rg % a.G, r = rg / a.G;
    const int64_t u = (int64_t)a.page_table[i] * a.G + g;
    const int at = atomicAdd(&cursor[u], 1);
    list[offs[u] + at] = r * a.nslot + s;
}

// Multi-workgroup counting sort (used while the G * P units fit an LDS
// histogram): workgroup w takes a contiguous chunk of the flattened (row,
// group, slot) selection, counts it per unit in LDS and writes its counts to
// row w of cnt[W][unit]; 16 threads per unit turn its column of cnt into an
// exclusive prefix over the workgroups (and the unit's total), the
// single-workgroup scan turns the totals into list offsets, and each workgroup
// places its chunk again with LDS cursors that start at offs[u] + cnt[w][u],
// so an entry's place in the list is one LDS atomic away.  Every global access
// of the three passes is coalesced, and there are no global atomics (the
// atomic inversion costs two contended global atomics per entry).
constexpr int kRemapThreads = 1024;
constexpr int kRemapMaxUnits = 16384;  // LDS histogram of 64 KB

__device__ __forceinline__ void remap_entry(const AttnArgs &a, int64_t i, int &r, int &g, int &s) {
    s = (int)(i % a.nslot);
    const int rg = (int)(i / a.nslot);
    g = rg % a.G;
    r = rg / a.G;
}

template <int HG>
__global__ __launch_bounds__(kRemapThreads) void remap_hist_kernel(AttnArgs a, int units, int W,
                                                                   int64_t chunk,
                                                                   int32_t *__restrict__ cnt) {
    __shared__ int32_t hist[kRemapMaxUnits];
    for (int u = threadIdx.x; u < units; u += kRemapThreads) hist[u] = 0;
    __syncthreads();
    const int w = blockIdx.x;
    const int64_t n = (int64_t)a.rows * a.G * a.nslot;
    const int64_t i1 = min(n, (w + 1) * chunk);
    for (int64_t i = w * chunk + threadIdx.x; i < i1; i += kRemapThreads) {
        int r, g, s;
        remap_entry(a, i, r, g, s);
        if (a.sel[i] < 0) {
            write_empty_slot<HG>(a, r, g, s, 0, 1);
            continue;
        }
        atomicAdd(&hist[a.page_table[i] * a.G + g], 1);
    }
    __syncthreads();
    for (int u = threadIdx.x; u < units; u += kRemapThreads) cnt[(int64_t)w * units + u] = hist[u];
}

// Exclusive prefix over the workgroups of every unit's column of cnt[W][unit],
// in place, and the unit totals: 16 units per workgroup and 16 threads per
// unit, each thread a run of up to 16 workgroup rows with all its loads in
// flight at once; the runs' sums are combined in LDS.  Needs W <= 256.
__global__ __launch_bounds__(256) void remap_unitscan_kernel(int units, int W,
                                                             int32_t *__restrict__ cnt,
                                                             int32_t *__restrict__ total) {
    __shared__ int part_sum[16][16];
    const int ul = threadIdx.x & 15, part = threadIdx.x >> 4;
    const int u = blockIdx.x * 16 + ul;
    const int rp = (W + 15) / 16;  // rows per run
    const int w0 = part * rp;
    int x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        x[i] = (u < units && i < rp && w0 + i < W) ? cnt[(int64_t)(w0 + i) * units + u] : 0;
    int run = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int v = x[i];
        x[i] = run;
        run += v;
    }
    part_sum[part][ul] = run;
    __syncthreads();
    int base = 0;
    for (int q = 0; q < part; ++q) base += part_sum[q][ul];
    if (u < units) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i < rp && w0 + i < W) cnt[(int64_t)(w0 + i) * units + u] = base + x[i];
        if (part == 15) total[u] = base + run;
    }
}

__global__ __launch_bounds__(kRemapThreads) void remap_place_kernel(
    AttnArgs a, int units, int W, int64_t chunk, const int32_t *__restrict__ cnt,
    const int32_t *__restrict__ offs, int32_t *__restrict__ list) {
    __shared__ int32_t cur[kRemapMaxUnits];
    const int w = blockIdx.x;
    for (int u = threadIdx.x; u < units; u += kRemapThreads)
        cur[u] = offs[u] + cnt[(int64_t)w * units + u];
    __syncthreads();
    const int64_t n = (int64_t)a.rows * a.G * a.nslot;
    const int64_t i1 = min(n, (w + 1) * chunk);
    for (int64_t i = w * chunk + threadIdx.x; i < i1; i += kRemapThreads) {
        if (a.sel[i] < 0) continue;
        int r, g, s;
        remap_entry(a, i, r, g, s);
        const int u = a.page_table[i] * a.G + g;
        list[atomicAdd(&cur[u], 1)] = r * a.nslot + s;
    }
}

template <int HG>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_blockmajor_kernel(
    AttnArgs a, const int32_t *__restrict__ offs, const int32_t *__restrict__ list,
    float scale_log2) {
    __shared__ AttnSmem sm;
    __shared__ __attribute__((aligned(16))) bf16_t ostage[kAttnWaves][8 * kStageRow];
    __shared__ int last_tok;
    const int64_t u = blockIdx.x;  // page * G + group
    const int o0 = offs[u], nq = offs[u + 1] - o0;
    if (nq == 0) return;
    const int g = (int)(u % a.G);
    const int64_t page = u / a.G;
    if (threadIdx.x == 0) last_tok = 0;
    KvStage st;
    stage_kv_load(st, a.k + page * a.kps + (int64_t)g * a.kgs, a.kts,
                  a.v + page * a.vps + (int64_t)g * a.vgs, a.vts);
    // the last token of the page that any query of the unit sees
    int mine = 0;
    for (int i = threadIdx.x; i < nq; i += kAttnThreads) {
        const int e = list[o0 + i];
        const int row = e / a.nslot, slot = e - row * a.nslot;
        const int blk = a.sel[((int64_t)row * a.G + g) * a.nslot + slot];
        mine = max(mine, min(kBlk - 1, a.row_pos[row] - blk * kBlk));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mine = max(mine, __shfl_xor(mine, m, kWave));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) atomicMax(&last_tok, mine);
    __syncthreads();
    stage_kv_store(sm, st, last_tok);
    __syncthreads();
    blockmajor_wave<HG>(sm, &ostage[threadIdx.x >> 6][0], a, g, list + o0, nq, scale_log2);
}

template <int HG>
__global__ __launch_bounds__(kDecThreads, DecComb<HG>::ml_in_slice ? 5 : 4) void attn_decode_kernel(
    AttnArgs a, float scale_log2) {
    __shared__ __attribute__((aligned(16))) char lds[4 * kWaveLds];
    const int unit = blockIdx.x;
    // the slot's block and page in one round trip (page -1 for an empty slot)
    const int blk = a.sel[unit];
    const int64_t page = a.page_table[unit];
    decode_unit<HG>(a, lds, unit, blk, page, scale_log2, threadIdx.x);
}

// Selection + page table + decode attention in one launch (select_unit, one
// workgroup per (row, group, slot)).
template <int HG, int KPT>
__global__ __launch_bounds__(kDecThreads, DecComb<HG>::ml_in_slice ? 5 : 4) void
attn_decode_select_kernel(AttnArgs a, SelectArgs sa, float scale_log2) {
    __shared__ __attribute__((aligned(16))) char lds[4 * kWaveLds];
    select_unit<HG, KPT>(a, sa, lds, blockIdx.x, scale_log2);
}

}  // namespace

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t stream) {
    const float sl2 = a.sm_scale * kLog2e;
    const dim3 grid((unsigned)((int64_t)a.rows * a.G * a.nslot)), block(kDecThreads);
    switch (a.Hg) {
        case 1: hipLaunchKernelGGL(attn_decode_kernel<1>, grid, block, 0, stream, a, sl2); break;
        case 2: hipLaunchKernelGGL(attn_decode_kernel<2>, grid, block, 0, stream, a, sl2); break;
        case 4: hipLaunchKernelGGL(attn_decode_kernel<4>, grid, block, 0, stream, a, sl2); break;
        case 8: hipLaunchKernelGGL(attn_decode_kernel<8>, grid, block, 0, stream, a, sl2); break;
        default: hipLaunchKernelGGL(attn_decode_kernel<16>, grid, block, 0, stream, a, sl2); break;
    }
    return hipGetLastError();
}

template <int KPT>
static void launch_decode_select_kpt(const AttnArgs &a, const SelectArgs &sa, float sl2,
                                     dim3 grid, dim3 block, hipStream_t stream) {
    switch (a.Hg) {
        case 1: hipLaunchKernelGGL((attn_decode_select_kernel<1, KPT>), grid, block, 0, stream, a, sa, sl2); break;
        case 2: hipLaunchKernelGGL((attn_decode_select_kernel<2, KPT>), grid, block, 0, stream, a, sa, sl2); break;
        case 4: hipLaunchKernelGGL((attn_decode_select_kernel<4, KPT>), grid, block, 0, stream, a, sa, sl2); break;
        case 8: hipLaunchKernelGGL((attn_decode_select_kernel<8, KPT>), grid, block, 0, stream, a, sa, sl2); break;
        default: hipLaunchKernelGGL((attn_decode_select_kernel<16, KPT>), grid, block, 0, stream, a, sa, sl2); break;
    }
}

// Workgroups of the fused kernel the device holds at once (one round), per
// device: the kernels of Hg <= 8 share one occupancy (LDS-bound), Hg = 16 keeps
// its maxima and sums in a separate LDS array and fits fewer.
int decode_select_capacity(int Hg) {
    static std::atomic<int> cap[64][2];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev < 0 || dev >= 64) dev = 0;
    const int v = Hg > 8 ? 1 : 0;
    int c = cap[dev][v].load(std::memory_order_relaxed);
    if (c == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        const hipError_t e =
            v ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &per_cu, attn_decode_select_kernel<16, 4>, kDecThreads, 0)
              : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &per_cu, attn_decode_select_kernel<8, 4>, kDecThreads, 0);
        if (e != hipSuccess) return 0;
        c = std::max(1, cus * per_cu);
        cap[dev][v].store(c, std::memory_order_relaxed);
    }
    return c;
}

hipError_t launch_attn_decode_select(const AttnArgs &a, const SelectArgs &sa,
                                     hipStream_t stream) {
    if (sa.score_stride > kSelectMaxBlocks) return hipErrorInvalidValue;
    const float sl2 = a.sm_scale * kLog2e;
    const dim3 grid((unsigned)((int64_t)a.rows * a.G * a.nslot)), block(kDecThreads);
    // scores per thread of the selecting workgroup
    if (sa.score_stride <= 2 * kDecThreads) launch_decode_select_kpt<2>(a, sa, sl2, grid, block, stream);
    else launch_decode_select_kpt<4>(a, sa, sl2, grid, block, stream);
    return hipGetLastError();
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups of the counting sort: about one selection entry per unit and
// workgroup (each workgroup also clears, writes and reads back one count per
// unit), at most 256 (one per CU); 0 selects the atomic inversion (units
// beyond the LDS histogram).
static int remap_workgroups(int64_t n, int64_t units) {
    if (units > kRemapMaxUnits) return 0;
    const int64_t w = n / (units + 1) + 1;
    return (int)std::min<int64_t>(256, w);
}

size_t prefill_workspace_bytes(int rows, int G, int nslot, int num_pages) {
    const size_t units = (size_t)G * num_pages;
    const int64_t n = (int64_t)rows * G * nslot;
    const int W = remap_workgroups(n, (int64_t)units);
    return align256(units * (size_t)std::max(W, 1) * 4) + align256(units * 4) +
           align256((units + 1) * 4) + align256((size_t)n * 4);
}

hipError_t launch_attn_prefill(const AttnArgs &a, int P, void *workspace, hipStream_t stream) {
    const int64_t units = (int64_t)a.G * P;
    const int64_t n = (int64_t)a.rows * a.G * a.nslot;
    const int W = remap_workgroups(n, units);
    char *ws = static_cast<char *>(workspace);
    int32_t *cnt = reinterpret_cast<int32_t *>(ws);
    ws += align256((size_t)units * std::max(W, 1) * 4);
    int32_t *counts = reinterpret_cast<int32_t *>(ws);
    ws += align256((size_t)units * 4);
    int32_t *offs = reinterpret_cast<int32_t *>(ws);
    ws += align256((size_t)(units + 1) * 4);
    int32_t *list = reinterpret_cast<int32_t *>(ws);
    const float sl2 = a.sm_scale * kLog2e;

#define MSA_BY_HG(KERNEL, GRID, BLOCK, ...)                                                      \
    switch (a.Hg) {                                                                              \
        case 1: hipLaunchKernelGGL(KERNEL<1>, GRID, BLOCK, 0, stream, __VA_ARGS__); break;       \
        case 2: hipLaunchKernelGGL(KERNEL<2>, GRID, BLOCK, 0, stream, __VA_ARGS__); break;       \
        case 4: hipLaunchKernelGGL(KERNEL<4>, GRID, BLOCK, 0, stream, __VA_ARGS__); break;       \
        case 8: hipLaunchKernelGGL(KERNEL<8>, GRID, BLOCK, 0, stream, __VA_ARGS__); break;       \
        default: hipLaunchKernelGGL(KERNEL<16>, GRID, BLOCK, 0, stream, __VA_ARGS__); break;     \
    }
    if (W > 0) {
        const int64_t chunk = (n + W - 1) / W;
        MSA_BY_HG(remap_hist_kernel, dim3(W), dim3(kRemapThreads), a, (int)units, W, chunk, cnt)
        hipLaunchKernelGGL(remap_unitscan_kernel, dim3((unsigned)((units + 15) / 16)), dim3(256),
                           0, stream, (int)units, W, cnt, counts);
        hipLaunchKernelGGL(remap_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts,
                           offs, (int)units);
        hipLaunchKernelGGL(remap_place_kernel, dim3(W), dim3(kRemapThreads), 0, stream, a,
                           (int)units, W, chunk, cnt, offs, list);
    } else {
        hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0,
                           stream, counts, units, 0);
        const dim3 eg((unsigned)((n + 255) / 256)), eb(256);
        MSA_BY_HG(remap_count_kernel, eg, eb, a, counts)
        hipLaunchKernelGGL(remap_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts,
                           offs, (int)units);
        hipLaunchKernelGGL(remap_scatter_kernel, eg, eb, 0, stream, a, counts, offs, list);
    }
#undef MSA_BY_HG
    const dim3 grid((unsigned)units), block(kAttnThreads);
    switch (a.Hg) {
        case 1: hipLaunchKernelGGL(attn_blockmajor_kernel<1>, grid, block, 0, stream, a, offs, list, sl2); break;
        case 2: hipLaunchKernelGGL(attn_blockmajor_kernel<2>, grid, block, 0, stream, a, offs, list, sl2); break;
        case 4: hipLaunchKernelGGL(attn_blockmajor_kernel<4>, grid, block, 0, stream, a, offs, list, sl2); break;
        case 8: hipLaunchKernelGGL(attn_blockmajor_kernel<8>, grid, block, 0, stream, a, offs, list, sl2); break;
        default: hipLaunchKernelGGL(attn_blockmajor_kernel<16>, grid, block, 0, stream, a, offs, list, sl2); break;
    }
    return hipGetLastError();
}

}  // namespace msa

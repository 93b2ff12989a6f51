// decode_dev.h -- the decode attention unit: one (row, KV group, slot)
// partial over one selected block, shared by the decode kernels (attn.hip) and
// the fused small-batch decode step (decode_fused.hip), so that both produce
// the same partials bit for bit (gfx950).
//
// Pages ("Together AI 解析如何高效服务 MiniMax M3"): dense attention of the query
// heads over the selected blocks (架构/特性), read through the per-group page
// table (将 MSA 与分页注意力集成).
#pragma once

#include "msa_internal.h"
#include "topk_select.h"

namespace msa {

// ------------------------------------------------------------------ decode
// One workgroup per (row, group, slot); its four waves split the 128-token
// block into 32-token slices, so every wave keeps loads in flight and the
// workgroup holds 32 KB of LDS (five fit on a CU: 1,280 resident units, a
// whole 8-row x 8-group x 17-slot decode step in one round).  Per wave:
//   K slice    straight from global into the 16x16x32 A operands (16 tokens x
//              32 dims per operand), non-temporal: each block is read once
//   V slice    global -> LDS without a register round trip (16 B per lane,
//              one 1 KB row group per instruction), then read back as V^T
//              operands with the gfx950 transposing LDS read, so V is never
//              scattered element by element
//   S^T = K Q^T, softmax local to the slice, O^T = V^T P^T (fp32 accumulate)
// and the four slices are combined in LDS the same way the final merge
// combines blocks (local maxima rescaled to the common one).  Slices that lie
// wholly past the row's position are neither loaded nor computed.
constexpr int kDecThreads = 256;
constexpr int kSlice = 32;             // tokens per wave
constexpr int kWaveLds = kSlice * 256;  // bytes per wave: its 32 x 256 B V slice
// After its P V a wave reuses its slice for the combine: un-normalised O^T as
// fp32 [head][dim] rows of comb_stride floats, then its row maxima and sums.
// With Hg <= 8 everything fits in the slice (32 KB of LDS per workgroup, five
// workgroups per CU); Hg = 16 keeps maxima and sums in a separate array.
template <int HG>
struct DecComb {
    static constexpr int stride = HG <= 8 ? 132 : 128;  // fp32; 132 spreads heads over banks
    static constexpr int ml_ofs = HG * stride * 4;      // byte offset of maxima, then sums
    static constexpr bool ml_in_slice = ml_ofs + 2 * 16 * 4 <= kWaveLds;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v4i16x2 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

// Lanes 16 c .. 16 c + 15 each name 8 bytes (4 dims) of a 4-token x 16-dim
// tile: lane s of the group points at token T0 + s / 4, dims D0 + 4 (s % 4).
// The transposing read hands lane i of the group dim D0 + i of tokens
// T0 .. T0 + 3 (element j = token T0 + j).
__device__ __forceinline__ v4i16 lds_read_tr(const char *lds_byte_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_byte_addr));
}

// Partial of one (row, group, slot) unit over block blk, cache page `page`,
// computed by a group of kDecThreads threads (gtid = thread index in the
// group, the group's four waves consecutive) with its own 32 KB of LDS at lds;
// an empty slot (blk < 0) or a block wholly past the row's position leaves an
// empty partial.  The function holds one workgroup barrier (between the
// slices and their combine).  A workgroup that is one group returns from an
// empty slot without it (the whole workgroup takes that path); with
// FULL_SYNC every path passes exactly one barrier, so that several groups of
// one workgroup can each run a unit of their own side by side.
template <int HG, bool FULL_SYNC = false>
__device__ __forceinline__ void decode_unit(const AttnArgs &a, char *lds, int unit, int blk,
                                            int64_t page, float scale_log2, int gtid) {
    using C = DecComb<HG>;
    // maxima and sums of wave i: ml(i)[0 .. 15] and ml(i)[16 .. 31]
    float *ml_extra = nullptr;
    if constexpr (!C::ml_in_slice) {
        __shared__ float ml_sep[4][32];
        ml_extra = &ml_sep[0][0];
    }
    auto ml = [&](int i) -> float * {
        if constexpr (C::ml_in_slice)
            return reinterpret_cast<float *>(lds + i * kWaveLds + C::ml_ofs);
        else
            return ml_extra + 32 * i;
    };
    const int s = unit % a.nslot;  // unit = (r, g, s)
    const int rg = unit / a.nslot;
    const int g = rg % a.G, r = rg / a.G;
    const int pos = a.row_pos[r];
    const int vis = pos - blk * kBlk;  // last visible token of the block
    if (blk < 0 || vis < 0) {
        write_empty_slot<HG>(a, r, g, s, gtid, kDecThreads);
        if constexpr (FULL_SYNC) __syncthreads();
        return;
    }
    const int H = a.G * HG;
    const int nact = min(4, vis / kSlice + 1);  // waves with a visible token
    const int lane = gtid & 63;
    const int w = __builtin_amdgcn_readfirstlane(gtid >> 6);
    const int c16 = lane & 15, grp = lane >> 4;
    char *wl_base = lds + w * kWaveLds;

    if (w < nact) {
        const int tok0 = w * kSlice;
        const bf16_t *kp = a.k + page * a.kps + (int64_t)g * a.kgs;
        const bf16_t *vp = a.v + page * a.vps + (int64_t)g * a.vgs;
        // V slice -> LDS, row-major [32 tokens][128 dims]: instruction i moves
        // tokens 4 i .. 4 i + 3, lane l 16 bytes (token 4 i + l / 16, dims 8 (l % 16))
#pragma unroll
        for (int i = 0; i < 8; ++i)
            __builtin_amdgcn_global_load_lds(vp + (int64_t)(tok0 + 4 * i + grp) * a.vts + 8 * c16,
                                             (lds_void *)(wl_base + 1024 * i), 16, 0, 0);
        // K operands: [tt][ks] = K[tok0 + 16 tt + l % 16][32 ks + 8 (l / 16) ..]
        bf16x8 kb[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                kb[tt][ks] = as_bf16x8(__builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                    kp + (int64_t)(tok0 + 16 * tt + c16) * a.kts + 32 * ks + 8 * grp)));
        // Q^T operands: head l % 16 (zero beyond Hg), dims 32 ks + 8 (l / 16) ..
        bf16x8 qb[4];
        const bf16_t *qp = a.q + ((int64_t)r * H + g * HG + (c16 < HG ? c16 : 0)) * 128 + 8 * grp;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[ks] = (c16 < HG) ? as_bf16x8(ld16(qp + 32 * ks)) : bf16x8{};

        // S^T tile tt: element i = token tok0 + 16 tt + 4 (l / 16) + i, head l % 16
        f32x4 st[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) st[tt] = mfma16(kb[tt][ks], qb[ks], st[tt]);
        float mx = -INFINITY;
        if (vis >= tok0 + kSlice - 1) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[tt][i]);
        } else {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = tok0 + 16 * tt + 4 * grp + i;
                    st[tt][i] = (tok <= vis) ? st[tt][i] : -INFINITY;
                    mx = fmaxf(mx, st[tt][i]);
                }
        }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);  // finite: token tok0 is visible
        const float off = -mx * scale_log2;
        float p[8], l = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[4 * tt + i] = __builtin_amdgcn_exp2f(fmaf(st[tt][i], scale_log2, off));
                l += p[4 * tt + i];
            }
        l = wave_sum_xor(l, 16);
        l = wave_sum_xor(l, 32);
        // P^T operand: K index 8 (l / 16) + i is token 4 (l / 16) + i of the slice,
        // 8 (l / 16) + 4 + i is token 16 + 4 (l / 16) + i
        u32x4 pw;
        pw[0] = pack_bf16x2(p[0], p[1]);
        pw[1] = pack_bf16x2(p[2], p[3]);
        pw[2] = pack_bf16x2(p[4], p[5]);
        pw[3] = pack_bf16x2(p[6], p[7]);
        const bf16x8 pb = as_bf16x8(pw);

        // the V slice has landed in LDS once this wave's loads are complete
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // masked tokens carry p = 0, but their cache rows may hold anything:
        // rows past the last visible token are cleared before they are read
        if (vis < tok0 + kSlice - 1) {
            for (int t = vis - tok0 + 1; t < kSlice; ++t)
                reinterpret_cast<uint32_t *>(wl_base + t * 256)[lane] = 0u;
        }
        // O^T tile dt: dims 16 dt + 4 (l / 16) + i, head l % 16
        f32x4 ot[8];
        const char *rd0 = wl_base + (4 * grp + (c16 >> 2)) * 256 + 8 * (c16 & 3);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const v4i16 lo = lds_read_tr(rd0 + 32 * dt);             // tokens 4 (l/16) + j
            const v4i16 hi = lds_read_tr(rd0 + 16 * 256 + 32 * dt);  // tokens 16 + 4 (l/16) + j
            const bf16x8 va = __builtin_bit_cast(
                bf16x8, v4i16x2{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
            ot[dt] = mfma16(va, pb, f32x4{});
        }
        // this wave's LDS now holds its un-normalised O^T, row max and sum
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (c16 < HG) {
            float *cb = reinterpret_cast<float *>(wl_base) + c16 * C::stride + 4 * grp;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4 *>(cb + 16 * dt) = ot[dt];
            if (grp == 0) {
                ml(w)[c16] = mx;
                ml(w)[16 + c16] = l;
            }
        }
    }
    __syncthreads();
    // combine: thread t owns head t / 16, dims 8 (t % 16) .. + 8
    const int t = gtid;
    if (t < HG * 16) {
        const int hh = t >> 4, c = t & 15;
        float m = ml(0)[hh];
        for (int i = 1; i < nact; ++i) m = fmaxf(m, ml(i)[hh]);
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        float L = 0.f;
        for (int i = 0; i < nact; ++i) {
            const float f = __builtin_amdgcn_exp2f((ml(i)[hh] - m) * scale_log2);
            L += f * ml(i)[16 + hh];
            const float *cb = reinterpret_cast<const float *>(lds + i * kWaveLds) +
                              hh * C::stride + 8 * c;
            const f32x4 x0 = *reinterpret_cast<const f32x4 *>(cb);
            const f32x4 x1 = *reinterpret_cast<const f32x4 *>(cb + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[e] += f * x0[e];
                acc[4 + e] += f * x1[e];
            }
        }
        const float inv = 1.f / L;
        const int64_t oi = ((int64_t)r * H + g * HG + hh) * a.nslot + s;
        u32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
        *reinterpret_cast<u32x4 *>(a.o_part + oi * 128 + 8 * c) = out;
        if (c == 0)
            a.lse_part[lse_index(a, r, s, g * HG + hh)] =
                (m * scale_log2 + __builtin_amdgcn_logf(L)) * kLn2;
    }
}

// Selection + page table + decode attention of one (row, group, slot) unit by a
// kDecThreads-thread workgroup with 32 KB of LDS at lds: every workgroup of a
// (row, group) runs the same top-k over the row's scores (exact integer
// decisions, so all of them agree), keeps its own slot's block, writes that
// slot of the selection and of the page table, and attends to it.  All four
// waves select, KPT scores per thread (0.9 us faster on a 64K-context batch
// than one wave with four times as many); the block-table entries of the
// candidates are read together with their scores, so the selected page is
// known as soon as the block is.  The selection's scratch lives in the LDS
// that the V slices use afterwards.
template <int HG, int KPT>
__device__ __forceinline__ void select_unit(const AttnArgs &a, const SelectArgs &sa, char *lds,
                                            int unit, float scale_log2) {
    using TS = TopkShared<kDecThreads / kWave>;
    static_assert(sizeof(TS) + 2 * sizeof(int) <= 4 * kWaveLds, "selection scratch");
    const int s = unit % a.nslot, rg = unit / a.nslot, r = rg / a.G;
    TS &sh = *reinterpret_cast<TS *>(lds);
    int *pick = reinterpret_cast<int *>(lds + sizeof(TS));
    {
        const int own = a.row_pos[r] / kBlk;
        const int req = sa.row_req ? sa.row_req[r] : r;
        const int32_t *bt = sa.block_table + (int64_t)req * sa.bt_stride;
        // block-table entries of the whole row, read with the scores (entries
        // past the request's last block are never used)
        const int n_bt = min(sa.score_stride, sa.bt_stride);
        int pg[KPT];
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int b = i * kDecThreads + (int)threadIdx.x;
            pg[i] = (b < n_bt) ? bt[b] : 0;
        }
        const int pg_own = bt[own];  // in flight while the selection runs
        topk_select_regs<kDecThreads, KPT>(
            sa.scores + (int64_t)rg * sa.score_stride, sa.score_stride, own, sa.k, sh,
            [&](int slot, int b, int i) {
                if (slot == s) {
                    int p = -1;
                    if (b >= 0) {
                        p = pg_own;
#pragma unroll
                        for (int j = 0; j < KPT; ++j) p = (j == i) ? pg[j] : p;
                    }
                    pick[0] = b;
                    pick[1] = p;
                }
            });
    }
    __syncthreads();
    const int blk = pick[0];
    const int64_t page = pick[1];
    if (threadIdx.x == 0) {
        sa.sel[unit] = blk;
        sa.page_table[unit] = (int32_t)page;
    }
    __syncthreads();  // the attention below reuses the selection's LDS
    decode_unit<HG>(a, lds, unit, blk, page, scale_log2, threadIdx.x);
}

}  // namespace msa

// topk_select.h -- radix selection of the top-k blocks of one (row, KV group),
// shared by the top-k kernels and the fused select + decode attention kernel
// (gfx950).
//
// Pages: the score part of MSA keeps the most relevant K blocks for each KV
// group (架构/特性 of "Together AI 解析如何高效服务 MiniMax M3"), with a top-k
// boundary per request and group (解码索引评分内核优化).  Ranking: score
// descending, ties to the lower block index; candidates are the blocks before
// the row's own block whose score is finite; the own block is appended after
// the kept ones; slots past it hold -1.
#pragma once

#include <type_traits>

#include "msa_internal.h"

namespace msa {

// Order-preserving key: larger float -> larger unsigned; -0 and +0 map together.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (f == 0.0f) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- wave-wide primitives on the VALU (DPP and the lane-swap ops; no LDS
// round trip, unlike a bpermute shuffle)

// op over the 64 lanes, the result in every lane: quad butterflies (l^1, l^2),
// the 8- and 16-lane mirrors (each pairs the two halves of the groups reduced
// so far), then the 16- and 32-lane swaps.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
    auto dpp = [](uint32_t x, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xf, 0xf,
                                                     false);
    };
    v = op(v, dpp(v, std::integral_constant<int, 0xb1>{}));   // quad_perm 1,0,3,2
    v = op(v, dpp(v, std::integral_constant<int, 0x4e>{}));   // quad_perm 2,3,0,1
    v = op(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
    v = op(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(p[0], p[1]);
    p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return op(p[0], p[1]);
}
__device__ __forceinline__ int wave_sum_i32(int v) {
    return (int)wave_reduce_u32((uint32_t)v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive prefix sum in lane order: shifts by 1, 2, 4, 8 within each 16-lane
// row (lanes without a source add 0), then lane 15 of rows 0 and 2 into rows 1
// and 3, then lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31
    return v;
}

// Barrier of the threads taking part in a selection: the workgroup barrier, or
// for a single wave only a wait for its own LDS operations (a wave's LDS
// operations complete in order, and the memory clobber keeps the compiler from
// moving loads or stores across).
template <int NW>
__device__ __forceinline__ void group_sync() {
    if constexpr (NW == 1)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    else
        __syncthreads();
}

// Exclusive prefix count of `flag` over the workgroup in thread order; returns
// the prefix for this thread and writes the workgroup total to *total.
template <int NWAVES = 4>
__device__ __forceinline__ int block_excl_count(bool flag, int *wave_tot, int *total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (NWAVES == 1) {
        *total = __popcll(bal);
        return in_wave;
    }
    if (lane == 0) wave_tot[w] = __popcll(bal);
    group_sync<NWAVES>();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) {
        const int c = wave_tot[i];
        before += (i < w) ? c : 0;
        tot += c;
    }
    group_sync<NWAVES>();
    *total = tot;
    return before + in_wave;
}

// Workgroup minimum and maximum of the valid (non-zero) keys: *lo = ~0u and
// *hi = 0 when there are none.  `xch` holds 2 * NWAVES words of LDS.
template <int NWAVES>
__device__ __forceinline__ void key_range(uint32_t lo, uint32_t hi, uint32_t *xch,
                                          uint32_t *lo_out, uint32_t *hi_out) {
    lo = wave_reduce_u32(lo, [](uint32_t a, uint32_t b) { return min(a, b); });
    hi = wave_reduce_u32(hi, [](uint32_t a, uint32_t b) { return max(a, b); });
    if (NWAVES > 1) {
        const int w = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) {
            xch[2 * w] = lo;
            xch[2 * w + 1] = hi;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NWAVES; ++i) {
            lo = min(lo, xch[2 * i]);
            hi = max(hi, xch[2 * i + 1]);
        }
        __syncthreads();
    }
    *lo_out = lo;
    *hi_out = hi;
}

// First digit shift of the radix select: the 8 bits that start at the highest
// bit where the smallest and largest candidate keys differ (the bits above it
// are common to every candidate and carry no rank information).  -1 when every
// candidate key is the same.
__device__ __forceinline__ int first_shift(uint32_t lo, uint32_t hi) {
    const uint32_t diff = lo ^ hi;
    if (diff == 0u) return -1;
    const int top = 31 - __clz((int)diff);
    return top > 7 ? top - 7 : 0;
}

// Digit d of the current radix pass such that the keys above it number fewer
// than `remain` and those at or above it at least `remain`; one wave scans the
// 256-bin histogram (4 bins per lane; the keys above a lane's bins are the
// total minus its inclusive prefix).
__device__ __forceinline__ void find_digit(const uint32_t *hist, int remain, int *digit,
                                           int *above_out) {
    const int lane = threadIdx.x & 63;
    const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
    const uint32_t h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
    const int local = (int)(h0 + h1 + h2 + h3);
    const int incl = wave_incl_scan(local);
    int above = __builtin_amdgcn_readlane(incl, kWave - 1) - incl;  // digits of higher lanes
    const int hd[4] = {(int)h0, (int)h1, (int)h2, (int)h3};
#pragma unroll
    for (int e = 3; e >= 0; --e) {
        if (above < remain && remain <= above + hd[e]) {
            *digit = 4 * lane + e;
            *above_out = above;
        }
        above += hd[e];
    }
}


// Workgroup scratch of the register-resident selection (LDS).
template <int NW>
struct TopkShared {
    uint32_t hist[256];
    int wave_tot[NW];
    uint32_t range_xch[2 * NW];
    int digit, above;
};

// Register-resident selection over the first `own` scores of one (row, group)
// with THREADS threads of the workgroup (all of them must call it; with THREADS
// = 64, one wave of a larger workgroup may call it alone), KPT keys per thread:
// block b = i * THREADS + tid, so the loads are coalesced and the ordered pass
// walks b in ascending order.  The whole score row (n_row entries) is loaded
// without waiting for `own`, so the loads overlap the read of the row's
// position; blocks from own on are masked afterwards.  8-bit radix passes on
// order-preserving keys (LDS histogram, one wave scans it) find the k-th
// largest key and how many keys equal to it are still needed; they start at the
// highest bit where the candidates' keys differ and stop once the bucket
// holding it is taken whole.  One ordered pass then keeps the keys above it
// plus the lowest-index keys equal to it and compacts them in ascending block
// order with ballots.  emit(slot, block, i) is called once for every slot
// 0 .. k, by one thread: i is the register index of a kept block of that
// thread, -1 for the own block and for the -1 padding.  Needs own < n_row <=
// KPT * THREADS and the scores s[0 .. n_row) readable.
template <int THREADS, int KPT, class Emit>
__device__ __forceinline__ void topk_select_regs(const float *__restrict__ s, int n_row, int own,
                                                 int k, TopkShared<THREADS / kWave> &sh,
                                                 Emit &&emit) {
    constexpr int NW = THREADS / kWave;
    const int tid = threadIdx.x;

    // key 0 marks "not a candidate"; every finite score's key is > 0
    uint32_t key[KPT];
    float raw[KPT];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int b = i * THREADS + tid;
        raw[i] = (b < n_row) ? s[b] : -INFINITY;
    }
    int nvalid = 0;
    uint32_t klo = ~0u, khi = 0u;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        const int b = i * THREADS + tid;
        const float v = (b < own) ? raw[i] : -INFINITY;
        key[i] = (v != -INFINITY) ? order_key(v) : 0u;
        nvalid += key[i] != 0u;
        klo = (key[i] != 0u) ? min(klo, key[i]) : klo;
        khi = max(khi, key[i]);
    }
    int ncand;
    {
        const int x = wave_sum_i32(nvalid);
        if (NW == 1) {
            ncand = x;
        } else {
            if ((tid & 63) == 0) sh.wave_tot[tid >> 6] = x;
            __syncthreads();
            ncand = 0;
#pragma unroll
            for (int i = 0; i < NW; ++i) ncand += sh.wave_tot[i];
            __syncthreads();
        }
    }

    // keep keys whose top bits (tmask) exceed thresh, plus the first take_eq
    // (in block order) whose top bits equal it
    uint32_t thresh = 0u, tmask = 0xffffffffu;
    int take_eq = 0;
    if (k == 0) {
        thresh = 0xffffffffu;
    } else if (k < ncand) {
        uint32_t lo, hi;
        key_range<NW>(klo, khi, sh.range_xch, &lo, &hi);
        uint32_t prefix = 0u, pmask = 0u;
        int remain = k;
        // digit passes from the highest differing bit down, 8 bits at a time; the
        // last one may overlap bits already fixed, which all counted keys share
        for (int shift = first_shift(lo, hi); shift >= 0; shift = shift > 8 ? shift - 8 : 0) {
            for (int i = tid; i < 256; i += THREADS) sh.hist[i] = 0u;
            group_sync<NW>();
#pragma unroll
            for (int i = 0; i < KPT; ++i)
                if (key[i] != 0u && (key[i] & pmask) == prefix)
                    atomicAdd(&sh.hist[(key[i] >> shift) & 255u], 1u);
            group_sync<NW>();
            if (tid < kWave) find_digit(sh.hist, remain, &sh.digit, &sh.above);
            group_sync<NW>();
            prefix |= (uint32_t)sh.digit << shift;
            pmask |= 255u << shift;
            remain -= sh.above;
            const bool whole_bucket = (int)sh.hist[sh.digit] == remain;
            group_sync<NW>();
            if (whole_bucket || shift == 0) break;  // selection decided
        }
        thresh = prefix;
        tmask = pmask;
        take_eq = remain;
    }

    int n_sel = 0, n_eq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
        if (i * THREADS >= own) break;  // uniform
        const int b = i * THREADS + tid;
        const bool valid = key[i] != 0u;
        const uint32_t kk = key[i] & tmask;
        const bool is_eq = valid && kk == thresh && take_eq > 0;
        int eq_tot;
        const int eq_rank = n_eq + block_excl_count<NW>(is_eq, sh.wave_tot, &eq_tot);
        const bool keep = valid && (kk > thresh || (is_eq && eq_rank < take_eq));
        int keep_tot;
        const int at = n_sel + block_excl_count<NW>(keep, sh.wave_tot, &keep_tot);
        if (keep) emit(at, b, i);
        n_sel += keep_tot;
        n_eq += eq_tot;
    }
    for (int i = n_sel + tid; i <= k; i += THREADS) emit(i, (i == n_sel) ? own : -1, -1);
}

}  // namespace msa

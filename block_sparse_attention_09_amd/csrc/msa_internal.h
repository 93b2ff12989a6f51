// msa_internal.h -- device helpers and launcher declarations shared by the
// libmsa translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa.h"

namespace msa {

constexpr int kBlk = 128;   // tokens per KV block and per cache page
constexpr int kWave = 64;   // CDNA wavefront

typedef uint16_t bf16_t;                                              // bf16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));            // MFMA A/B operand
typedef float f32x4 __attribute__((ext_vector_type(4)));              // 16x16 accumulator
typedef float f32x16 __attribute__((ext_vector_type(16)));            // 32x32 accumulator
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));           // 16-byte load

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l holds A[l % 16][8 (l / 16) .. +8], B[8 (l / 16) .. +8][l % 16] and
// D[4 (l / 16) + i][l % 16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l holds A[l % 32][8 (l / 32) .. +8], B[8 (l / 32) .. +8][l % 32] and
// D[8 q + 4 (l / 32) + r][l % 32] in element 4 q + r (q, r = 0..3).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// v combined with its value in lane l ^ mask, the result in every lane.  For
// mask 16 and 32 the partner values come from the gfx950 lane-swap VALU ops
// (v_permlane16_swap exchanges the odd 16-lane rows of one operand with the even
// rows of the other, v_permlane32_swap the upper half of one with the lower half
// of the other: with both operands v, the two results hold v and v at l ^ mask),
// which stay off the LDS pipe that a bpermute shuffle goes through; both lanes
// of a pair combine the same two values, so they agree bit for bit.
__device__ __forceinline__ float2 xor_partners(float v, int mask) {
    const uint32_t u = __float_as_uint(v);
    if (mask == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return make_float2(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    if (mask == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return make_float2(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    return make_float2(v, __shfl_xor(v, mask, kWave));
}
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    const float2 p = xor_partners(v, mask);
    return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float wave_sum_xor(float v, int mask) {
    const float2 p = xor_partners(v, mask);
    return p.x + p.y;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are validated by the API layer.
hipError_t launch_index_score(const msa_dims_t &d, int rows, const bf16_t *q_idx,
                              const msa_view_t &kv, const int32_t *block_table, int bt_stride,
                              const int32_t *row_req, const int32_t *row_pos,
                              const int32_t *blk_lo, int num_reqs, float *scores,
                              int score_stride, hipStream_t stream);

// With page_table != nullptr the page of every selected block is written too
// (block_table[row_req[r]][sel], -1 for empty slots).
// Prefill shape (many rows per request): the row-tiled scorer.
hipError_t launch_index_score_tiled(const msa_dims_t &d, int rows, const bf16_t *q_idx,
                                    const msa_view_t &kv, const int32_t *block_table,
                                    int bt_stride, const int32_t *row_req, const int32_t *row_pos,
                                    const int32_t *blk_lo, float *scores, int score_stride,
                                    hipStream_t stream);

hipError_t launch_topk(int rows, int G, const float *scores, int score_stride,
                       const int32_t *row_pos, int k, int32_t *sel, hipStream_t stream,
                       const int32_t *row_req = nullptr, const int32_t *block_table = nullptr,
                       int bt_stride = 0, int32_t *page_table = nullptr);

hipError_t launch_page_table(int rows, int G, const int32_t *sel, int nslot,
                             const int32_t *row_req, const int32_t *block_table, int bt_stride,
                             int32_t *page_table, hipStream_t stream);

struct AttnArgs {
    int rows, G, Hg, nslot;
    const bf16_t *q;
    const bf16_t *k;
    int64_t kps, kgs, kts;
    const bf16_t *v;
    int64_t vps, vgs, vts;
    const int32_t *sel, *page_table, *row_pos;
    float sm_scale;
    bf16_t *o_part;
    float *lse_part;
};

// Index of the LSE of (row r, slot s, head h) in lse_part [rows][nslot][H]:
// the heads of one (row, slot) are contiguous, so the Hg LSEs a (row, group,
// slot) produces land in one sector instead of Hg scattered ones.
__device__ __forceinline__ int64_t lse_index(const AttnArgs &a, int r, int s, int h) {
    return ((int64_t)r * a.nslot + s) * (a.G * a.Hg) + h;
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
        if (ch == 0) a.lse_part[lse_index(a, r, s, g * HG + hh)] = -INFINITY;
    }
}

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t stream);

// Top-k + page table + decode attention in one launch (sel, page_table written
// by the kernel; a.sel / a.page_table unused).  Scores per (row, group) at most
// kSelectMaxBlocks.  decode_select_capacity(Hg) is the number of its workgroups
// the device holds at once (0 if the query fails).
struct SelectArgs {
    const float *scores;
    int score_stride, k;
    const int32_t *row_req, *block_table;
    int bt_stride;
    int32_t *sel, *page_table;
};
constexpr int kSelectMaxBlocks = 1024;
hipError_t launch_attn_decode_select(const AttnArgs &a, const SelectArgs &sa, hipStream_t stream);
int decode_select_capacity(int Hg);

// The whole decode step in one launch (decode_fused.hip): the streaming scan,
// selection, page table, slot partials and their merge, synchronised through
// sync, int32 [kStepSyncHead + 2 * rows * G] (zero on entry, zero again when
// the kernel ends; word 2 is set to 1 if a wait ever hit its poll bound).
// a.sel / a.page_table are unused (f.sel / f.page_table are written).
// Supported for d_idx 64 or 128 and score_stride <= kSelectMaxBlocks.
struct StepArgs {
    int n_idx;
    const bf16_t *q_idx, *kidx;
    int64_t kips, kigs, kits;
    const int32_t *block_table;
    int bt_stride;
    const int32_t *row_req, *blk_lo;
    float *scores;
    int score_stride, k;
    int32_t *sel, *page_table;
    bf16_t *o;
    float *lse;
    float index_scale;  // 1 / sqrt(d_idx)
    int32_t *sync;
    int nscan_waves, spin_limit;  // set by launch_decode_step
};
constexpr int kStepSyncHead = 4;
bool decode_step_supported(int d_idx, int score_stride);
hipError_t launch_decode_step(const AttnArgs &a, StepArgs f, int d_idx, hipStream_t stream);

size_t prefill_workspace_bytes(int rows, int G, int nslot, int num_pages);

// Scratch of the allocation-free prefill entry point: a static device array of
// this many bytes (MSA_NOALLOC_SCRATCH_BYTES in msa.h); noalloc_scratch gives
// its address on the current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = MSA_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_attn_prefill(const AttnArgs &a, int num_pages, void *workspace,
                               hipStream_t stream);

hipError_t launch_lse_merge(int rows, int H, int nslot, const bf16_t *o_part,
                            const float *lse_part, bf16_t *o, float *lse, hipStream_t stream);

// copy of the selected K/V pages into a compact device pool (decoupled offload)
hipError_t launch_gather_pages(int rows, int G, int nslot, const int32_t *page_table,
                               const msa_view_t &k, const msa_view_t &v, bf16_t *dst_k,
                               bf16_t *dst_v, int32_t *dst_page_table, hipStream_t stream);

// measured-peak probes (not part of the MSA path)
hipError_t launch_peak_stream_read(const void *buf, int64_t bytes, float *sink,
                                   hipStream_t stream);
hipError_t launch_peak_stream_write(void *buf, int64_t bytes, uint32_t tag, hipStream_t stream);
hipError_t launch_peak_row_copy(const void *src, void *dst, const int32_t *load_idx,
                                const int32_t *store_idx, int64_t n, int tiles_per_wg,
                                int layout, hipStream_t stream);
hipError_t launch_peak_mfma_bf16(int iters, float *sink, double *flops, hipStream_t stream);
hipError_t launch_peak_mfma_bf16_random(int iters, float *sink, double *flops,
                                       hipStream_t stream);

}  // namespace msa

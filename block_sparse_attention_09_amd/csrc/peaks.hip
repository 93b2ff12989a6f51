// peaks.hip -- measured machine peaks (gfx950), the reference points the MSA
// kernels' rooflines are read against besides the published ones: a plain
// streaming read of a large buffer (HBM), a streaming write (whose bytes a read
// right after may find in the last-level cache) and register-resident bf16 MFMA loops
// (matrix cores), one on fixed low-entropy operands and one on pseudo-random
// operands of unit variance like the MSA workloads' values: the matrix cores'
// sustained rate depends on the operand bits they toggle (the chip lowers its
// rate under the higher power draw of random data).  None is part of the MSA
// path.
#include "msa_internal.h"

namespace msa {

namespace {

constexpr int kPeakThreads = 256;

// Workgroup w reads the contiguous 64 KB chunk w of the buffer, every thread
// keeping eight non-temporal 16-B loads in flight (the fastest of the grid
// shapes and depths tried on MI355X), and folds what it read into one word;
// the fold is stored only if it equals a value no sane input produces, which
// keeps every load alive at the cost of nothing.
constexpr int64_t kReadChunk16 = (64 << 10) / 16;  // 16-B units per workgroup
constexpr int kReadDepth = 8;

__global__ __launch_bounds__(kPeakThreads) void stream_read_kernel(const u32x4 *__restrict__ p,
                                                                   int64_t n16,
                                                                   float *__restrict__ sink) {
    const int64_t b = (int64_t)blockIdx.x * kReadChunk16;
    const int64_t e = b + kReadChunk16 < n16 ? b + kReadChunk16 : n16;
    uint32_t acc = 0u;
    int64_t i = b + threadIdx.x;
    for (; i + (kReadDepth - 1) * kPeakThreads < e; i += kReadDepth * kPeakThreads) {
        u32x4 v[kReadDepth];
#pragma unroll
        for (int k = 0; k < kReadDepth; ++k)
            v[k] = __builtin_nontemporal_load(p + i + k * kPeakThreads);
#pragma unroll
        for (int k = 0; k < kReadDepth; ++k) acc += v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    for (; i < e; i += kPeakThreads) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    if (acc == 0x9e3779b9u) sink[0] = __uint_as_float(acc);
}

// Streaming write of the same shape: workgroup w writes its 64 KB chunk, every
// thread storing eight 16-B values per round (cached stores, so a read of the
// same bytes right after can find them in the last-level cache).
__global__ __launch_bounds__(kPeakThreads) void stream_write_kernel(u32x4 *__restrict__ p,
                                                                    int64_t n16, uint32_t tag) {
    const int64_t b = (int64_t)blockIdx.x * kReadChunk16;
    const int64_t e = b + kReadChunk16 < n16 ? b + kReadChunk16 : n16;
    for (int64_t i = b + threadIdx.x; i < e; i += kPeakThreads) {
        const uint32_t x = tag ^ (uint32_t)i;
        p[i] = u32x4{x, x + 1u, x + 2u, x + 3u};
    }
}

// Four independent 32x32x16 bf16 accumulation chains per wave, operands in
// registers: the matrix-core rate with nothing else in the way.
__global__ __launch_bounds__(kPeakThreads) void mfma_loop_kernel(int iters,
                                                                 float *__restrict__ sink) {
    bf16x8 a, b[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)threadIdx.x + (float)e);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j][e] = (__bf16)(0.5f * (float)e - (float)j);
    }
    f32x16 c[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = mfma32(a, b[j], c[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += c[j][j];
    if (s == 1.2345f) sink[0] = s;
}

// Pseudo-random operands: each lane holds 8 A and 8 B fragments of roughly
// normal bf16 values (a sum of four uniforms from an integer hash of the lane,
// fragment and element), and two accumulation chains cycle through them, so
// consecutive MFMAs see different random operands as a real contraction does.
__device__ __forceinline__ uint32_t peak_hash(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__device__ __forceinline__ float peak_normalish(uint32_t key) {
    const uint32_t h0 = peak_hash(key), h1 = peak_hash(key ^ 0x5bd1e995u);
    const float u = (float)(h0 & 0xffff) + (float)(h0 >> 16) + (float)(h1 & 0xffff) +
                    (float)(h1 >> 16);
    // four uniforms on [0, 65536): mean 131070, variance 4 * 65536^2 / 12
    return (u - 131070.f) * (1.7320508f / 65536.f);
}

__global__ __launch_bounds__(kPeakThreads) void mfma_random_loop_kernel(int iters,
                                                                        float *__restrict__ sink) {
    const uint32_t t = blockIdx.x * kPeakThreads + threadIdx.x;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[i][e] = (__bf16)peak_normalish((t * 8u + i) * 16u + e);
            b[i][e] = (__bf16)peak_normalish((t * 8u + i) * 16u + 8u + e + 0x40000000u);
        }
    f32x16 c0 = {}, c1 = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c0 = mfma32(a[i], b[i], c0);
#pragma unroll
        for (int i = 0; i < 8; ++i) c1 = mfma32(a[i], b[(i + 3) & 7], c1);
    }
    const float s = c0[0] + c1[1];
    if (s == 1.2345f) sink[0] = s;
}

// Row gather-scatter: the memory pattern of the block-major prefill kernel
// without its arithmetic.  A workgroup takes `tpw` consecutive tiles of 32
// rows of 256 bytes, its four waves one tile each in turn; a wave loads its
// tile's 32 source rows (cached loads: four whole rows per instruction, or 32
// rows x 32 bytes per instruction, the layout of 32 MFMA operand rows), passes
// them through its own LDS stage (rows padded by 16 bytes) and stores four
// whole rows per instruction to the destination rows, non-temporally.  The
// next tile's loads are issued before the current tile's stores; the row
// indices of all of a wave's tiles are loaded up front (at most 16 tiles per
// wave), so no wait for a row index has to wait for earlier stores.
constexpr int kCopyMaxTilesPerWg = 64;
constexpr int kCopyStageRow = 17;  // 16-B chunks per staged row (16 + 1 pad)

__global__ __launch_bounds__(kPeakThreads) void row_copy_kernel(
    const bf16_t *__restrict__ src, bf16_t *__restrict__ dst, const int32_t *__restrict__ lidx,
    const int32_t *__restrict__ sidx, int64_t ntiles, int tpw, int layout) {
    __shared__ u32x4 stage[kPeakThreads / kWave][32 * kCopyStageRow];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t t0 = (int64_t)blockIdx.x * tpw;
    const int64_t t1 = t0 + tpw < ntiles ? t0 + tpw : ntiles;
    const int nmine = t0 + w < t1 ? (int)((t1 - t0 - w + 3) / 4) : 0;  // <= 16
    if (nmine == 0) return;
    // row indices of this wave's tiles k = 0 .. nmine - 1 (tile t0 + w + 4 k):
    // lane l holds row l % 32 of each
    int li[kCopyMaxTilesPerWg / 4], si[kCopyMaxTilesPerWg / 4];
#pragma unroll
    for (int k = 0; k < kCopyMaxTilesPerWg / 4; ++k) {
        const int64_t e = (t0 + w + 4 * k) * 32 + (lane & 31);
        li[k] = k < nmine ? lidx[e] : 0;
        si[k] = k < nmine ? sidx[e] : 0;
    }
    u32x4 *st = &stage[w][0];
    auto load_tile = [&](int row_here, u32x4 (&v)[8]) {
        if (layout == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = __shfl(row_here, 4 * i + (lane >> 4), kWave);
                v[i] = ld16(src + (int64_t)row * 128 + 8 * (lane & 15));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = ld16(src + (int64_t)row_here * 128 + 16 * i + 8 * (lane >> 5));
        }
    };
    u32x4 v[8];
    load_tile(li[0], v);
#pragma unroll
    for (int k = 0; k < kCopyMaxTilesPerWg / 4; ++k) {
        if (k >= nmine) continue;  // wave-uniform
        // stage row r of the tile at st[r * kCopyStageRow + chunk]
        if (layout == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) st[(4 * i + (lane >> 4)) * kCopyStageRow + (lane & 15)] = v[i];
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) st[(lane & 31) * kCopyStageRow + 2 * i + (lane >> 5)] = v[i];
        }
        if (k + 1 < kCopyMaxTilesPerWg / 4 && k + 1 < nmine) load_tile(li[k + 1], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = 4 * i + (lane >> 4);
            const int row = __shfl(si[k], r, kWave);
            __builtin_nontemporal_store(st[r * kCopyStageRow + (lane & 15)],
                                        reinterpret_cast<u32x4 *>(dst + (int64_t)row * 128 +
                                                                  8 * (lane & 15)));
        }
    }
}

}  // namespace

hipError_t launch_peak_row_copy(const void *src, void *dst, const int32_t *load_idx,
                                const int32_t *store_idx, int64_t n, int tiles_per_wg,
                                int layout, hipStream_t stream) {
    const int64_t ntiles = n / 32;
    const int64_t grid = (ntiles + tiles_per_wg - 1) / tiles_per_wg;
    hipLaunchKernelGGL(row_copy_kernel, dim3((unsigned)grid), dim3(kPeakThreads), 0, stream,
                       static_cast<const bf16_t *>(src), static_cast<bf16_t *>(dst), load_idx,
                       store_idx, ntiles, tiles_per_wg, layout);
    return hipGetLastError();
}

hipError_t launch_peak_stream_read(const void *buf, int64_t bytes, float *sink,
                                   hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + kReadChunk16 - 1) / kReadChunk16;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kPeakThreads), 0, stream,
                       static_cast<const u32x4 *>(buf), n16, sink);
    return hipGetLastError();
}

hipError_t launch_peak_stream_write(void *buf, int64_t bytes, uint32_t tag, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t grid = (n16 + kReadChunk16 - 1) / kReadChunk16;
    hipLaunchKernelGGL(stream_write_kernel, dim3((unsigned)grid), dim3(kPeakThreads), 0, stream,
                       static_cast<u32x4 *>(buf), n16, tag);
    return hipGetLastError();
}

hipError_t launch_peak_mfma_bf16(int iters, float *sink, double *flops, hipStream_t stream) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int grid = 2 * cus;  // two workgroups per CU: two waves per SIMD
    *flops = (double)grid * (kPeakThreads / kWave) * (double)iters * 4.0 * (2.0 * 32 * 32 * 16);
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(kPeakThreads), 0, stream, iters, sink);
    return hipGetLastError();
}

hipError_t launch_peak_mfma_bf16_random(int iters, float *sink, double *flops,
                                       hipStream_t stream) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int grid = 2 * cus;  // two workgroups per CU: two waves per SIMD
    *flops = (double)grid * (kPeakThreads / kWave) * (double)iters * 16.0 * (2.0 * 32 * 32 * 16);
    hipLaunchKernelGGL(mfma_random_loop_kernel, dim3(grid), dim3(kPeakThreads), 0, stream, iters,
                       sink);
    return hipGetLastError();
}

}  // namespace msa

// bpw_dense_head.hip - dense bfloat16 head GEMV with float32 accumulation.
//
// Written for CDNA4 (wave64); launched only by bpw_host.cpp after its argument and architecture
// checks.
#include "bpw_device.h"

namespace bpw {

// Dense bf16 head GEMV: one wave per row group of kHeadRows rows; x staged once per workgroup in
// LDS; each lane streams 16-byte chunks (8 bf16) and accumulates in fp32 with v_dot2c_f32_bf16.

constexpr int kHeadRows = 4;   // rows a wave works on at once

// a.lo * b.lo + a.hi * b.hi + c over bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16). The words
// arrive by value: bit-casting a vector component in place reads the wrong element with this
// compiler, so components are always copied into scalars first.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
constexpr int kHeadIters = 4;  // row groups per wave per workgroup

__global__ __launch_bounds__(kThreads) void dense_head_kernel(const uint16_t *__restrict__ w, int64_t rows,
                                                              int64_t cols, const uint16_t *__restrict__ x,
                                                              float *__restrict__ y) {
    extern __shared__ uint32_t lds[];
    const int nchunk = (int)(cols / 8);
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(x);
    u32x4 *lx = reinterpret_cast<u32x4 *>(lds);
    for (int i = threadIdx.x; i < nchunk; i += kThreads) lx[i] = xs[i];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t rbase = (int64_t)blockIdx.x * (kWaves * kHeadIters * kHeadRows);
    for (int it = 0; it < kHeadIters; ++it) {
        const int64_t r0 = rbase + (int64_t)(it * kWaves + wave) * kHeadRows;
        float acc[kHeadRows];
        const u32x4 *wr[kHeadRows];
        bool ok[kHeadRows];
#pragma unroll
        for (int i = 0; i < kHeadRows; ++i) {
            acc[i] = 0.0f;
            ok[i] = (r0 + i) < rows;
            wr[i] = reinterpret_cast<const u32x4 *>(w + (ok[i] ? (r0 + i) : 0) * cols);
        }
        for (int c = lane; c < nchunk; c += 64) {
            const u32x4 xv = lx[c];
            u32x4 wv[kHeadRows];
#pragma unroll
            for (int i = 0; i < kHeadRows; ++i) wv[i] = __builtin_nontemporal_load(wr[i] + c);
#pragma unroll
            for (int i = 0; i < kHeadRows; ++i) {
                acc[i] = dot2_bf16(wv[i].x, xv.x, acc[i]);
                acc[i] = dot2_bf16(wv[i].y, xv.y, acc[i]);
                acc[i] = dot2_bf16(wv[i].z, xv.z, acc[i]);
                acc[i] = dot2_bf16(wv[i].w, xv.w, acc[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < kHeadRows; ++i) {
            float v = acc[i];
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            v += __shfl_xor(v, 4);
            v += __shfl_xor(v, 8);
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            if (lane == 0 && ok[i]) y[r0 + i] = v;
        }
    }
}

// ------------------------------------------------------------------------------------------
// Launchers.

int launch_dense_head(const uint16_t *w, int64_t rows, int64_t cols, const uint16_t *x, float *y, void *stream) {
    if (rows <= 0) return hipSuccess;
    const int64_t per_wg = (int64_t)kWaves * kHeadIters * kHeadRows;
    const unsigned grid = (unsigned)((rows + per_wg - 1) / per_wg);
    const size_t lds = (size_t)cols * 2;
    hipLaunchKernelGGL(dense_head_kernel, dim3(grid), dim3(kThreads), lds, as_stream(stream), w, rows, cols, x, y);
    return hipGetLastError();
}

}  // namespace bpw

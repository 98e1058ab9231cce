// bpw_dense_head.hip - dense bfloat16 head GEMV with float32 accumulation.
//
// Written for CDNA4 (wave64); launched only by bpw_host.cpp after its argument and architecture
// checks.
#include "bpw_device.h"

namespace bpw {

// Dense bf16 head GEMV (Tritium paper, "Where the bytes are": the head is the largest single tensor a
// decode step reads). Each wave owns kHeadRows consecutive rows; a lane streams 16-byte chunks (8
// bf16) c = lane, lane + 64, ... of every one of them and accumulates in fp32 with v_dot2c_f32_bf16,
// then a wave butterfly sums the lanes. x (a few KB) is read through the cache by every lane, with
// no staging or barrier. Small workgroups (kWaves * kHeadRows = 8 rows) keep the tail of the launch
// short. For 2560-column rows the five chunks a lane reads per row are compile-time, so all of its
// loads are issued before the first is used. Workgroup b runs on XCD b mod (XCD count), so blocks are
// renumbered to give each XCD one contiguous run of rows. Measured at 128256 x 2560: 99.1 us with x
// staged in LDS and 64 rows per workgroup, 93.6-93.9 us in this form with rows in launch order, 91.9
// us with the XCD runs (7.1 TB/s).

constexpr int kHeadRows = 2;  // rows of one wave

// a.lo * b.lo + a.hi * b.hi + c over bf16 pairs, fp32 accumulate (v_dot2c_f32_bf16). The words
// arrive by value: bit-casting a vector component in place reads the wrong element with this
// compiler, so components are always copied into scalars first.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float dot8_bf16(const u32x4 &w, const u32x4 &x, float acc) {
    acc = dot2_bf16(w.x, x.x, acc);
    acc = dot2_bf16(w.y, x.y, acc);
    acc = dot2_bf16(w.z, x.z, acc);
    return dot2_bf16(w.w, x.w, acc);
}

// NCH > 0: every row has exactly 64 * NCH chunks (cols == 512 * NCH); NCH == 0: any cols % 8 == 0.
template <int NCH>
__global__ __launch_bounds__(kThreads) void dense_head_kernel(const uint16_t *__restrict__ w, int64_t rows,
                                                              int64_t cols, const uint16_t *__restrict__ x,
                                                              float *__restrict__ y, int xcds) {
    const int64_t nchunk = cols / 8;
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(x);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // workgroup b runs on XCD b mod xcds: give each XCD one contiguous run of row blocks
    const int64_t nb = gridDim.x, b = blockIdx.x, xc = b % xcds, per = nb / xcds, extra = nb % xcds;
    const int64_t lb = xc * per + (xc < extra ? xc : extra) + b / xcds;
    const int64_t r0 = (lb * kWaves + wave) * kHeadRows;
    float acc[kHeadRows];
    const u32x4 *wr[kHeadRows];
    bool ok[kHeadRows];
#pragma unroll
    for (int i = 0; i < kHeadRows; ++i) {
        acc[i] = 0.0f;
        ok[i] = (r0 + i) < rows;
        wr[i] = reinterpret_cast<const u32x4 *>(w + (ok[i] ? (r0 + i) : 0) * cols);  // past the end: row 0, unused
    }
    if constexpr (NCH > 0) {
        u32x4 xv[NCH], wv[NCH][kHeadRows];
#pragma unroll
        for (int k = 0; k < NCH; ++k) xv[k] = xs[lane + 64 * k];
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int i = 0; i < kHeadRows; ++i) wv[k][i] = __builtin_nontemporal_load(wr[i] + lane + 64 * k);
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int i = 0; i < kHeadRows; ++i) acc[i] = dot8_bf16(wv[k][i], xv[k], acc[i]);
    } else {
        for (int64_t c = lane; c < nchunk; c += 64) {
            const u32x4 xv = xs[c];
            u32x4 wv[kHeadRows];
#pragma unroll
            for (int i = 0; i < kHeadRows; ++i) wv[i] = __builtin_nontemporal_load(wr[i] + c);
#pragma unroll
            for (int i = 0; i < kHeadRows; ++i) acc[i] = dot8_bf16(wv[i], xv, acc[i]);
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

// ------------------------------------------------------------------------------------------
// Launchers.

int launch_dense_head(const uint16_t *w, int64_t rows, int64_t cols, const uint16_t *x, float *y, void *stream) {
    const int xcds = host_xcds();
    if (rows <= 0) return hipSuccess;
    const int64_t per_wg = (int64_t)kWaves * kHeadRows;
    const unsigned grid = (unsigned)((rows + per_wg - 1) / per_wg);
    if (cols == 2560)
        hipLaunchKernelGGL(dense_head_kernel<5>, dim3(grid), dim3(kThreads), 0, as_stream(stream), w, rows, cols, x, y,
                           xcds);
    else
        hipLaunchKernelGGL(dense_head_kernel<0>, dim3(grid), dim3(kThreads), 0, as_stream(stream), w, rows, cols, x, y,
                           xcds);
    return hipGetLastError();
}

}  // namespace bpw

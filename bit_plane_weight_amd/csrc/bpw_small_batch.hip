// bpw_small_batch.hip - small-batch ternary GEMM: each beat read once and applied to every token.
//
// Written for CDNA4 (wave64); launched only by bpw_host.cpp after its argument and architecture
// checks.
#include "bpw_device.h"

namespace bpw {

// Small-batch activation planes: a token-major batch X [batch][ldx] -> [batch][bpr][16] words, word
// 2j + h of a block holding bit j of its columns 32h .. 32h+31 (the batch-1 GEMV's order), one wave
// per 64-column block (eight ballots give the eight planes).
__global__ __launch_bounds__(kThreads) void stage_batch_kernel(const int8_t *__restrict__ X, int64_t ldx,
                                                               uint32_t *__restrict__ xplanes, int32_t bpr,
                                                               int32_t batch) {
    const int item = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (item >= bpr * batch) return;
    const int lane = threadIdx.x & 63;
    const int t = item / bpr, b = item - t * bpr;
    const uint32_t xv = (uint8_t)X[(int64_t)t * ldx + (int64_t)b * 64 + lane];
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint64_t m = __ballot((xv >> j) & 1u);
        if ((lane >> 1) == j) word = (lane & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
    }
    if (lane < 16) xplanes[((int64_t)t * bpr + b) * 16 + lane] = word;
}

// ------------------------------------------------------------------------------------------
// Small-batch GEMM, bit-serial: each beat is loaded once and applied to every token. The batch's
// activation planes sit in LDS ([batch][bpr][16] words); lanes of one row group read the same
// block addresses, so reads across row groups of a wave are broadcasts.

template <int K>
__device__ __forceinline__ void gemm_sb_tile(const SmallBatchArgs &A, const uint32_t *lds, int row0, int lane,
                                             int wave) {
    const int glog = A.glog;
    const int G = 1 << glog;
    const int g = lane & (G - 1);
    const int q = lane >> glog;
    const int rpi = 64 >> glog;
    const int bpr = A.bpr;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(A.planes, (uint32_t)((uint64_t)A.rows * bpr * 16));
    const u32x4 *lx = reinterpret_cast<const u32x4 *>(lds);

    for (int it = 0; it < kIters; ++it) {
        const int row = row0 + (it * kWaves + wave) * rpi + q;
        for (int ch = 0; ch < A.nchunk; ++ch) {
            const int bbase = ch * K * G + g;
            u32x4 v[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int b = bbase + k * G;
                const uint32_t off = (b < bpr) ? (uint32_t)(((uint32_t)row * (uint32_t)bpr + (uint32_t)b) * 16u)
                                               : kOutOfRange;
                v[k] = load_beat(wr, off);
            }
            uint32_t cn = 0;
#pragma unroll
            for (int k = 0; k < K; ++k) {
                cn = __builtin_popcount(v[k].z) + cn;
                cn = __builtin_popcount(v[k].w) + cn;
            }
            for (int t = 0; t < A.batch; ++t) {
                uint32_t c[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const int b = bbase + k * G;
                    const int bb = b < bpr ? b : 0;  // v[k] is zero past bpr, any planes give 0
                    uint32_t X[16];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const u32x4 w = lx[((t * bpr) + bb) * 4 + i];
                        X[4 * i + 0] = w.x;
                        X[4 * i + 1] = w.y;
                        X[4 * i + 2] = w.z;
                        X[4 * i + 3] = w.w;
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        c[j] = __builtin_popcount(select_bits(X[2 * j], v[k].x, v[k].z)) + c[j];
                        c[j] = __builtin_popcount(select_bits(X[2 * j + 1], v[k].y, v[k].w)) + c[j];
                    }
                }
                int32_t acc = (int32_t)cn;
#pragma unroll
                for (int j = 0; j < 7; ++j) acc += (int32_t)(c[j] << j);
                acc -= (int32_t)(c[7] << 7);
                const int32_t tot = group_sum(acc, glog);
                if (g == 0 && row < A.rows) {
                    int32_t *o = A.out_i32 + (int64_t)t * A.rows + row;
                    const int32_t prev = (ch == 0) ? 0 : *o;
                    const int32_t val = prev + tot;
                    *o = val;
                    if (ch + 1 == A.nchunk && A.out_f32) {
                        float f = (float)val * A.x_scales[t];
                        A.out_f32[(int64_t)t * A.rows + row] = f * A.w_scale;
                    }
                }
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void gemm_small_batch_kernel(SmallBatchArgs A) {
    extern __shared__ uint32_t lds[];
    const int words = A.batch * A.bpr * 16;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(A.xplanes);
    u32x4 *dst = reinterpret_cast<u32x4 *>(lds);
    for (int i = threadIdx.x; i < words / 4; i += kThreads) dst[i] = src[i];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row0 = blockIdx.x * A.tile_rows;
    switch (A.kblk) {
        case 1: gemm_sb_tile<1>(A, lds, row0, lane, wave); break;
        case 2: gemm_sb_tile<2>(A, lds, row0, lane, wave); break;
        case 3: gemm_sb_tile<3>(A, lds, row0, lane, wave); break;
        case 4: gemm_sb_tile<4>(A, lds, row0, lane, wave); break;
        case 5: gemm_sb_tile<5>(A, lds, row0, lane, wave); break;
        case 6: gemm_sb_tile<6>(A, lds, row0, lane, wave); break;
        case 7: gemm_sb_tile<7>(A, lds, row0, lane, wave); break;
        default: {
            for (int it = 0; it < kIters; ++it) {
                const int row = row0 + (it * kWaves + wave) * 64 + lane;
                if (row < A.rows)
                    for (int t = 0; t < A.batch; ++t) {
                        A.out_i32[(int64_t)t * A.rows + row] = 0;
                        if (A.out_f32) A.out_f32[(int64_t)t * A.rows + row] = 0.0f * A.x_scales[t] * A.w_scale;
                    }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Launchers.

int launch_stage_batch(const int8_t *X, int64_t ldx, uint32_t *xplanes, int32_t bpr, int32_t batch, void *stream) {
    const int64_t items = (int64_t)bpr * batch;
    if (items <= 0) return hipSuccess;
    const unsigned grid = (unsigned)((items + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(stage_batch_kernel, dim3(grid), dim3(kThreads), 0, as_stream(stream), X, ldx, xplanes, bpr,
                       batch);
    return hipGetLastError();
}

int launch_gemm_small_batch(const SmallBatchArgs &a, int32_t n_tiles, void *stream) {
    if (n_tiles <= 0) return hipSuccess;
    const size_t lds = (size_t)a.batch * a.bpr * 64;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_small_batch_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(gemm_small_batch_kernel, dim3((unsigned)n_tiles), dim3(kThreads), lds, as_stream(stream), a);
    return hipGetLastError();
}

}  // namespace bpw

// bpw_bytelane.hip - batch-1 grouped ternary GEMV, byte-lane select (a pinned alternative to the bit-serial kernel).
//
// Written for CDNA4 (wave64); launched only by bpw_host.cpp after its argument and architecture
// checks.
#include "bpw_device.h"

namespace bpw {

// Batch-1 GEMV, byte-lane select: each 4-bit group of a mask is widened to four byte lanes
// (n * 0x00204081 places bit i at bit 7i; & 0x01010101 keeps bits 0, 8, 16, 24) and a signed
// 4-way int8 dot product (v_dot4_i32_i8) accumulates x over the +1 and the -1 lanes separately.
// Same tiling as the bit-serial kernel; lanes keep x itself (16 words per block) in registers.

__device__ __forceinline__ int32_t spread4(uint32_t m, int i) {
    return (int32_t)((((m >> (4 * i)) & 0xFu) * 0x00204081u) & 0x01010101u);
}

template <int K>
__device__ __forceinline__ void gemv_bytelane_tile(const DevJob &J, int row0, int lane, int wave) {
    const int glog = J.glog;
    const int G = 1 << glog;
    const int g = lane & (G - 1);
    const int q = lane >> glog;
    const int rpi = 64 >> glog;
    const int bpr = J.bpr;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(J.planes, (uint32_t)((uint64_t)J.rows * bpr * 16));
    const u32x4 *__restrict__ xq = reinterpret_cast<const u32x4 *>(J.x);

    for (int ch = 0; ch < J.nchunk; ++ch) {
        const int bbase = ch * K * G + g;
        int32_t X[K][16];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int b = bbase + k * G;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (b < bpr) v = xq[b * 4 + i];
                X[k][4 * i + 0] = (int32_t)v.x;
                X[k][4 * i + 1] = (int32_t)v.y;
                X[k][4 * i + 2] = (int32_t)v.z;
                X[k][4 * i + 3] = (int32_t)v.w;
            }
        }
        int32_t s[kIters];
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int row = row0 + (it * kWaves + wave) * rpi + q;
            u32x4 v[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int b = bbase + k * G;
                const uint32_t off = (b < bpr) ? (uint32_t)(((uint32_t)row * (uint32_t)bpr + (uint32_t)b) * 16u)
                                               : kOutOfRange;
                v[k] = load_beat(wr, off);
            }
            int32_t ap = 0, an = 0;
#pragma unroll
            for (int k = 0; k < K; ++k) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    ap = __builtin_amdgcn_sdot4(spread4(v[k].x, i), X[k][i], ap, false);
                    an = __builtin_amdgcn_sdot4(spread4(v[k].z, i), X[k][i], an, false);
                    ap = __builtin_amdgcn_sdot4(spread4(v[k].y, i), X[k][8 + i], ap, false);
                    an = __builtin_amdgcn_sdot4(spread4(v[k].w, i), X[k][8 + i], an, false);
                }
            }
            s[it] = ap - an;
        }
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int row = row0 + (it * kWaves + wave) * rpi + q;
            const int32_t tot = group_sum(s[it], glog);
            if (g == 0 && row < J.rows) {
                if (J.nchunk == 1) {
                    write_row(J, job_x_scale(J), row, tot);
                } else {
                    const int32_t prev = (ch == 0) ? 0 : J.out_i32[row];
                    if (ch + 1 < J.nchunk)
                        J.out_i32[row] = prev + tot;
                    else
                        write_row(J, job_x_scale(J), row, prev + tot);
                }
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void gemv_bytelane_kernel(const DevJob *__restrict__ jobs,
                                                                 const DevTile *__restrict__ tiles) {
    const DevTile tile = tiles[blockIdx.x];
    const DevJob J = jobs[tile.job];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    switch (J.kblk) {
        case 1: gemv_bytelane_tile<1>(J, tile.row0, lane, wave); break;
        case 2: gemv_bytelane_tile<2>(J, tile.row0, lane, wave); break;
        case 3: gemv_bytelane_tile<3>(J, tile.row0, lane, wave); break;
        case 4: gemv_bytelane_tile<4>(J, tile.row0, lane, wave); break;
        case 5: gemv_bytelane_tile<5>(J, tile.row0, lane, wave); break;
        case 6: gemv_bytelane_tile<6>(J, tile.row0, lane, wave); break;
        case 7: gemv_bytelane_tile<7>(J, tile.row0, lane, wave); break;
        default: {
            for (int it = 0; it < kIters; ++it) {
                const int row = tile.row0 + (it * kWaves + wave) * 64 + lane;
                if (row < J.rows) write_row(J, job_x_scale(J), row, 0);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Launchers.

int launch_gemv_tiles(const DevJob *jobs, const DevTile *tiles, int32_t n_tiles, void *stream) {
    if (n_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_bytelane_kernel, dim3((unsigned)n_tiles), dim3(kThreads), 0, as_stream(stream), jobs,
                       tiles);
    return hipGetLastError();
}

}  // namespace bpw

// bpw_gemv_tokens.hip - grouped GEMV for 2 to 4 tokens at once (small batch), bit-serial, gfx950.
//
// The batch-1 kernel's stream and select (Tritium paper, introduction, Equations 2-3, and "On
// popcount"; beats as in "The .trit format, version 1", 2.3) with NT activation vectors: every beat
// is loaded once and reduced against each token's bit planes in turn, so the weight bytes per step do
// not grow with the batch while the select work does (NT x 34 VALU per beat). Same tile table as the
// batch-1 grouped GEMV (one job per tile, tiles laid out per XCD), same two-register-set streaming
// loop and LDS row-group claiming; the planes of all NT tokens sit in LDS side by side. Served shapes
// are the model's two row widths (2560 and 6912 columns); the host sends other shapes to the
// matrix-core kernel. Launched only by bpw_host.cpp after its argument and architecture checks.
#include <hip/hip_runtime.h>

#include "bpw_device.h"

namespace bpw {

namespace {

__device__ __forceinline__ int tok_claim(uint32_t *claim, int lane) {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(claim, 1u);
    return (int)__builtin_amdgcn_readfirstlane(v);
}

}  // namespace

// Row-groups u0 .. u1-1 of the job (64 / G rows each), all NT tokens. Row sums collect in LDS and
// leave in one coalesced pass per token at the end (a store inside the loop would count against the
// vector-memory counter the weight loads use).
template <int NT, int K, int GLOG, int NB>
__device__ __forceinline__ void tok_tile(const TokJob &J, int u0, int u1, int wave, int lane, u32x4 (*xl)[kXPassBlocks * 4],
                                         int32_t (*sums)[kTokTileRows], uint32_t *claim) {
    constexpr int G = 1 << GLOG;
    constexpr int rpi = 64 >> GLOG;
    const int g = lane & (G - 1);
    const int q = lane >> GLOG;
    const int n = u1 - u0;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(J.planes, J.plane_bytes);
    auto issue = [&](u32x4 (&B)[K], int v) {
        issue_row<K, NB>(B, wr, (uint32_t)((u0 + v) * rpi + q), v < n, g, G, NB);
    };
    u32x4 B0[K], B1[K];
    int v = wave;  // every wave's first row-group is fixed; the rest are claimed
    issue(B0, v);
    if (threadIdx.x == 0) *claim = (uint32_t)kWaves;
#pragma unroll
    for (int t = 0; t < NT; ++t) stage_planes(xl[t], J.X + (int64_t)t * J.ldx, 0, NB, wave, lane);
    __syncthreads();
    // As in the batch-1 kernel: one trip handles two row-groups with every load issued on every path
    // (row-groups past the tile read zeros and store nothing), so the waits cover the older set only.
    while (v < n) {
        const int va = tok_claim(claim, lane);
        issue(B1, va);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int32_t tot = group_sum(row_partial<K, GLOG>(xl[t], B0, g, G), GLOG);
            if (g == 0) sums[t][v * rpi + q] = tot;
        }
        const int vb = tok_claim(claim, lane);
        issue(B0, vb);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int32_t tot = group_sum(row_partial<K, GLOG>(xl[t], B1, g, G), GLOG);
            if (g == 0 && va < n) sums[t][va * rpi + q] = tot;
        }
        v = vb;
    }
    __syncthreads();
    const int row0 = u0 * rpi, nr = n * rpi;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const float xs = J.x_scales[t];
        for (int i = threadIdx.x; i < nr; i += kThreads) {
            const int row = row0 + i;
            if (row < J.rows) {
                const int64_t idx = (int64_t)t * J.rows + row;
                const int32_t s = sums[t][i];
                J.out_i32[idx] = s;
                if (J.out_f32) J.out_f32[idx] = ((float)s * xs) * J.w_scale;  // the scales in turn
            }
        }
    }
}

template <int NT>
__global__ __launch_bounds__(kThreads) void gemv_tokens_kernel(const TokJob *__restrict__ jobs,
                                                               const Tile *__restrict__ tiles) {
    __shared__ u32x4 xl[NT][kXPassBlocks * 4];
    __shared__ int32_t sums[NT][kTokTileRows];
    __shared__ uint32_t claim;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Tile t = tiles[blockIdx.x];
    const TokJob J = jobs[t.job];
    if (J.bpr == 40)  // 2560-column rows: 8 lanes x 5 beats
        tok_tile<NT, 5, 3, 40>(J, t.u0, t.u1, wave, lane, xl, sums, &claim);
    else  // 6912-column rows: 32 lanes x 4 beats (108 of 128 used)
        tok_tile<NT, 4, 5, 108>(J, t.u0, t.u1, wave, lane, xl, sums, &claim);
}

int launch_gemv_tokens(const TokJob *jobs, const Tile *tiles, int32_t n_tiles, int32_t nt, void *stream) {
    if (n_tiles <= 0) return hipSuccess;
    const dim3 grid((unsigned)n_tiles), block(kThreads);
    switch (nt) {
        case 2: hipLaunchKernelGGL(gemv_tokens_kernel<2>, grid, block, 0, as_stream(stream), jobs, tiles); break;
        case 3: hipLaunchKernelGGL(gemv_tokens_kernel<3>, grid, block, 0, as_stream(stream), jobs, tiles); break;
        case 4: hipLaunchKernelGGL(gemv_tokens_kernel<4>, grid, block, 0, as_stream(stream), jobs, tiles); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bpw

// bpw_small_batch.hip - small-batch ternary GEMM on gfx950: out[t][r] = sum_c W[r][c] * X[t][c].
//
// The batch-1 select-accumulate (Tritium paper, introduction, Equations 2-3) applied to a few
// tokens at once. A wave loads its row-group's beats once and reuses them for every token of its
// token group, so the weights stream from HBM once per call whatever the batch. Written for CDNA4
// (wave64, 160 KB LDS); launched only by bpw_host.cpp after its argument and architecture checks.
//
// Grid: blockIdx.x picks kSBWaves consecutive row-groups (one per wave), blockIdx.y a group of up to
// A.tg tokens. The workgroup builds its tokens' activation planes in LDS straight from X (token t of
// the group at xl + t * kXPassBlocks * 4, the batch-1 word order and block rotation), so a call is a
// single launch.
#include "bpw_device.h"

namespace bpw {

// Planes of tokens [t0, t0 + nt), blocks [b0, b0 + nb) of X into LDS, all threads of the workgroup;
// one 16-byte piece per lane per round. Each lane uses its load inside the branch that issued it.
__device__ __forceinline__ void stage_tokens(u32x4 *xl, const int8_t *X, int64_t ldx, int t0, int nt, int b0,
                                             int nb) {
    const int per_token = nb * 4;
    const int total = nt * per_token;
    uint16_t *xh = reinterpret_cast<uint16_t *>(xl);
    for (int base = 0; base < total; base += kSBThreads) {
        const int p = base + (int)threadIdx.x;
        if (p < total) {
            const int t = p / per_token, pp = p - t * per_token;
            const u32x4 v =
                *reinterpret_cast<const u32x4 *>(X + (int64_t)(t0 + t) * ldx + (int64_t)b0 * 64 + (int64_t)pp * 16);
            uint32_t pl[8];
            piece_planes(v.x, v.y, v.z, v.w, pl);
            const int b = pp >> 2, qq = pp & 3;
            const int tbase = t * kXPassBlocks * 4;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int w = 2 * j + (qq >> 1);
                xh[((tbase + xq_slot(b, w >> 2)) * 4 + (w & 3)) * 2 + (qq & 1)] = (uint16_t)pl[j];
            }
        }
    }
}

// One wave's row-group rg for tokens [t0, t0 + nt). Rows past the matrix read zeros and store
// nothing. Wide rows (several passes) add each pass into the output the same lane wrote before.
template <int K, int GLOG, int NB>
__device__ __forceinline__ void sb_rowgroup(const SmallBatchArgs &A, u32x4 *xl, int rg, int t0, int nt, int lane) {
    const int glog = GLOG >= 0 ? GLOG : A.glog;
    const int G = 1 << glog;
    const int g = lane & (G - 1);
    const int q = lane >> glog;
    const int rpi = 64 >> glog;
    const int bpr = NB > 0 ? NB : A.bpr;
    const int pass_blocks = K * G;
    const int nchunk = NB > 0 ? 1 : A.nchunk;
    const int row = rg * rpi + q;
    const bool live = row < A.rows;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(A.planes, A.plane_bytes);
    for (int ch = 0; ch < nchunk; ++ch) {
        const int b0 = ch * pass_blocks;
        const int nb = min(pass_blocks, bpr - b0);
        u32x4 B[K];
        issue_row<K, NB>(B, wr, (uint32_t)row, live, b0 + g, G, bpr);
        __syncthreads();  // the previous pass's planes are no longer read
        stage_tokens(xl, A.X, A.ldx, t0, nt, b0, nb);
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            const int32_t tot = group_sum(row_partial<K, GLOG>(xl + t * kXPassBlocks * 4, B, g, G), glog);
            if (live && g == 0) {
                const int64_t idx = (int64_t)(t0 + t) * A.rows + row;
                const int32_t val = ch == 0 ? tot : A.out_i32[idx] + tot;
                A.out_i32[idx] = val;
                if (ch + 1 == nchunk && A.out_f32) {
                    const float f = (float)val * A.x_scales[t0 + t];  // exact integer times the token's scale
                    A.out_f32[idx] = f * A.w_scale;                  // then the weight scale
                }
            }
        }
    }
}

__global__ __launch_bounds__(kSBThreads) void gemm_small_batch_kernel(SmallBatchArgs A) {
    extern __shared__ u32x4 xl[];  // A.tg tokens x kXPassBlocks blocks x 4 quarters
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = blockIdx.x * kSBWaves + wave;
    const int t0 = blockIdx.y * A.tg;
    const int nt = min(A.tg, A.batch - t0);
    if (A.bpr == 40) {  // 2560-column rows: 8 lanes x 5 beats
        sb_rowgroup<5, 3, 40>(A, xl, rg, t0, nt, lane);
    } else if (A.bpr == 108) {  // 6912-column rows: 32 lanes x 4 beats
        sb_rowgroup<4, 5, 108>(A, xl, rg, t0, nt, lane);
    } else if (A.kblk == 0) {  // no columns: every sum is empty (row-groups of 64 rows)
        const int row = rg * 64 + lane;
        if (row < A.rows)
            for (int t = 0; t < nt; ++t) {
                const int64_t idx = (int64_t)(t0 + t) * A.rows + row;
                A.out_i32[idx] = 0;
                if (A.out_f32) A.out_f32[idx] = (0.0f * A.x_scales[t0 + t]) * A.w_scale;
            }
    } else if (A.kblk == 1) {
        sb_rowgroup<1, -1, 0>(A, xl, rg, t0, nt, lane);
    } else {
        sb_rowgroup<2, -1, 0>(A, xl, rg, t0, nt, lane);
    }
}

// ------------------------------------------------------------------------------------------
// Launcher.

int launch_gemm_small_batch(const SmallBatchArgs &a, int32_t row_wgs, int32_t token_groups, void *stream) {
    if (row_wgs <= 0 || token_groups <= 0) return hipSuccess;
    const size_t lds = (size_t)a.tg * kXPassBlocks * 64;
    if (lds > 64 * 1024) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_small_batch_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(gemm_small_batch_kernel, dim3((unsigned)row_wgs, (unsigned)token_groups), dim3(kSBThreads), lds,
                       as_stream(stream), a);
    return hipGetLastError();
}

}  // namespace bpw

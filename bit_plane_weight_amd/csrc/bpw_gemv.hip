// bpw_gemv.hip - batch-1 grouped ternary GEMV (bit-serial select) for gfx950.
//
// Written for CDNA4 (wave64, 4 SIMDs per CU, 160 KB LDS); launched only by bpw_host.cpp after its
// argument and architecture checks.
//
// Batch-1 select-accumulate (Tritium paper, introduction, Equations 2-3). Weights stream as
// .trit v1 beats ("The .trit format, version 1", 2.3): 16 bytes = pos[64] | neg[64]. With the
// activation split into its eight two's-complement bit planes X_j (Tritium paper, "On popcount"),
// the exact row sum is
//     acc = sum_j w_j * (popc(pos & X_j) - popc(neg & X_j)),   w_j = 2^j (j < 7), w_7 = -128.
// Because pos and neg are disjoint (P1), f_j = (pos & X_j) | (neg & ~X_j) is one 3-input bitwise
// select (v_bitop3_b32), and popc(f_j) = popc(pos & X_j) + popc(neg) - popc(neg & X_j). Summing
// with the weights w_j, whose total is -1, gives
//     acc = sum_j w_j * popc(f_j) + popc(neg)
// so one beat costs 16 selects + 18 accumulating popcounts (v_bcnt_u32_b32) for both planes,
// against ~128 ops for widening mask bits to byte lanes. Padding bits are clear (P2), so whole
// 64-column blocks are processed with no tail loop; the sum is an exact integer, so lane order and
// reduction order cannot change it (Tritium paper, "Verification").
#include <hip/hip_runtime.h>

#include "bpw_gemv_tile.h"

namespace bpw {

__global__ __launch_bounds__(kThreads) void gemv_bitserial_kernel(const DevJob *__restrict__ jobs,
                                                                  const Tile *__restrict__ tiles) {
    __shared__ u32x4 xl[kXPassBlocks * 4];
    __shared__ int32_t sums[kTileRows];
    __shared__ uint32_t claim;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Tile t = tiles[blockIdx.x];
    const DevJob &J = jobs[t.job];  // read where used: the tile record feeds the first loads
    bs_dispatch<false>(J, t, wave, lane, xl, sums, &claim);
}

// ------------------------------------------------------------------------------------------
// Launchers.

int launch_gemv_bitserial(const DevJob *jobs, const Tile *tiles, int32_t n_tiles, void *stream) {
    if (n_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_bitserial_kernel, dim3((unsigned)n_tiles), dim3(kThreads), 0, as_stream(stream), jobs,
                       tiles);
    return hipGetLastError();
}

}  // namespace bpw

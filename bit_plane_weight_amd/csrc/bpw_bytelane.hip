// bpw_bytelane.hip - batch-1 grouped ternary GEMV, byte-lane select (a pinned alternative to the
// bit-serial kernel of bpw_gemv.hip).
//
// Written for CDNA4 (wave64); launched only by bpw_host.cpp after its argument and architecture
// checks. It runs the bit-serial kernel's tiles, XCD layout, two-set prefetch loop, reduction and
// output pass unchanged (bpw_gemv_tile.h); only the select differs: x is staged as bytes, and each
// beat's masks are widened to byte lanes and dotted with x by v_dot4_i32_i8 (row_partial_bytelane),
// the masked-byte formulation of "The .trit format, version 1", section 1.
#include <hip/hip_runtime.h>

#include "bpw_gemv_tile.h"

namespace bpw {

__global__ __launch_bounds__(kThreads) void gemv_bytelane_kernel(const DevJob *__restrict__ jobs,
                                                                 const Tile *__restrict__ tiles) {
    __shared__ u32x4 xl[kXPassBlocks * 4];
    __shared__ int32_t sums[kTileRows];
    __shared__ uint32_t claim;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Tile t = tiles[blockIdx.x];
    const DevJob &J = jobs[t.job];  // read where used: the tile record feeds the first loads
    bs_dispatch<true>(J, t, wave, lane, xl, sums, &claim);
}

int launch_gemv_bytelane(const DevJob *jobs, const Tile *tiles, int32_t n_tiles, void *stream) {
    if (n_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_bytelane_kernel, dim3((unsigned)n_tiles), dim3(kThreads), 0, as_stream(stream), jobs,
                       tiles);
    return hipGetLastError();
}

}  // namespace bpw

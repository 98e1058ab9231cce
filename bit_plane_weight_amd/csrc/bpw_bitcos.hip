// bpw_bitcos.hip - batch-1 grouped GEMV on BITCOS matrices for gfx950.
//
// BITCOS ("BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits", "A bitmap and a sign")
// stores a presence bit per weight and a sign bit per nonzero, compacted in column order. A block of
// 64 columns is decoded back to the pos/neg planes of the .trit beat: the block's signs start after
// the nonzeros of the row's earlier blocks, so each lane finds its sign offset with a prefix
// popcount across the row's lanes, reads a 64-bit window of the row's sign words, and deposits the
// window's bits into the presence positions (neg), four positions at a time through a 256-entry LDS
// table (presence nibble | four sign bits -> the nibble's neg bits); pos = presence & ~neg. The
// select-accumulate of the batch-1 kernel then runs on those planes unchanged. Launched only by
// bpw_bitcos_host.cpp after its argument and architecture checks.
#include <hip/hip_runtime.h>

#include "bpw_device.h"

namespace bpw {

// Table entry i: the bits of nibble p = i & 15 set where p is set, taken in order from s = i >> 4.
__device__ __forceinline__ uint8_t deposit_entry(uint32_t i) {
    const uint32_t p = i & 15u, s = i >> 4;
    uint32_t out = 0, k = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if ((p >> b) & 1u) {
            out |= ((s >> k) & 1u) << b;
            ++k;
        }
    }
    return (uint8_t)out;
}

// The low popc(p) bits of s deposited into the set positions of p (32 bits).
__device__ __forceinline__ uint32_t deposit32(const uint8_t *lut, uint32_t p, uint32_t s) {
    uint32_t neg = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t p4 = (p >> (4 * t)) & 15u;
        neg |= (uint32_t)lut[p4 | ((s & 15u) << 4)] << (4 * t);
        s >>= __builtin_popcount(p4);
    }
    return neg;
}

// Inclusive sum over the lanes g' <= g of an aligned group of 8 lanes (DPP row shifts stay inside the
// group for the lanes that add them).
__device__ __forceinline__ uint32_t scan8(uint32_t v, int g) {
    uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    if (g >= 1) v += t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    if (g >= 2) v += t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    if (g >= 4) v += t;
    return v;
}

// Row-groups [u0, u1) of 8 rows: lanes g = 0..7 of a row hold blocks g, g + 8, ... (K of them; past
// bpr they read zeros); wave w takes row-groups u0 + w, u0 + w + kWaves, ...
template <int K>
__device__ __forceinline__ void bc_tile(const BitcosJob &J, int u0, int u1, int wave, int lane, const u32x4 *xl,
                                        const uint8_t *lut) {
    const int g = lane & 7, q = lane >> 3;
    const int bpr = J.bpr;
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(J.presence, J.presence_bytes);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(J.row_start, J.row_start_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(J.signs, J.sign_bytes);
    const float xs = J.x_scale;
    for (int u = u0 + wave; u < u1; u += kWaves) {
        const int row = u * 8 + q;
        const bool live = row < J.rows;
        uint32_t plo[K], phi[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const int b = g + 8 * k;
            const uint32_t off = (live && b < bpr) ? ((uint32_t)row * (uint32_t)bpr + (uint32_t)b) * 8u : kOutOfRange;
            const uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(pr, off, 0, kAuxNT));
            plo[k] = (uint32_t)v;
            phi[k] = (uint32_t)(v >> 32);
        }
        const uint32_t rs = __builtin_amdgcn_raw_buffer_load_b32(rr, live ? (uint32_t)row * 4u : kOutOfRange, 0, 0);
        // sign windows: block k's signs start after the row's nonzeros in earlier blocks
        u32x4 w[K];
        uint32_t sh_k[K];
        uint32_t done = 0;  // nonzeros of the row in the block sets before k
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t c = (uint32_t)__builtin_popcount(plo[k]) + (uint32_t)__builtin_popcount(phi[k]);
            const uint32_t o = done + scan8(c, g) - c;
            const uint32_t off = (live && c != 0) ? (rs + (o >> 5)) * 4u : kOutOfRange;
            w[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, off, 0, 0));
            sh_k[k] = o & 31u;
            done += (uint32_t)group_sum((int32_t)c, 3);
        }
        u32x4 B[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const uint32_t sh = sh_k[k];
            const uint64_t win = (uint64_t)w[k].x | ((uint64_t)w[k].y << 32);
            const uint64_t s = sh ? ((win >> sh) | ((uint64_t)w[k].z << (64 - sh))) : win;
            const uint32_t nlo = deposit32(lut, plo[k], (uint32_t)s);
            const uint32_t nhi = deposit32(lut, phi[k], (uint32_t)(s >> __builtin_popcount(plo[k])));
            B[k] = u32x4{plo[k] & ~nlo, phi[k] & ~nhi, nlo, nhi};
        }
        const int32_t tot = group_sum(row_partial<K, 3>(xl, B, g, 8), 3);
        if (g == 0 && live) {
            J.out_i32[row] = tot;
            if (J.out_f32) J.out_f32[row] = ((float)tot * xs) * J.w_scale;  // the scales in turn
        }
    }
}

__global__ __launch_bounds__(kThreads) void gemv_bitcos_kernel(const BitcosJob *__restrict__ jobs,
                                                               const Tile *__restrict__ tiles) {
    __shared__ u32x4 xl[kXPassBlocks * 4];
    __shared__ uint8_t lut[256];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Tile t = tiles[blockIdx.x];
    const BitcosJob J = jobs[t.job];
    lut[threadIdx.x] = deposit_entry(threadIdx.x);  // 256 threads, 256 entries
    stage_planes(xl, J.x, 0, J.bpr, wave, lane);
    __syncthreads();
    if (J.bpr == 40)
        bc_tile<5>(J, t.u0, t.u1, wave, lane, xl, lut);
    else if (J.bpr == 108)
        bc_tile<14>(J, t.u0, t.u1, wave, lane, xl, lut);
    else
        bc_tile<16>(J, t.u0, t.u1, wave, lane, xl, lut);
}

int launch_gemv_bitcos(const BitcosJob *jobs, const Tile *tiles, int32_t n_tiles, void *stream) {
    if (n_tiles <= 0) return hipSuccess;
    static_assert(kThreads == 256, "one table entry per thread");
    hipLaunchKernelGGL(gemv_bitcos_kernel, dim3((unsigned)n_tiles), dim3(kThreads), 0, as_stream(stream), jobs, tiles);
    return hipGetLastError();
}

}  // namespace bpw

// bpw_device.h - device-side helpers shared by the gfx950 kernels of libbpw (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include "bpw_internal.h"

namespace bpw {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource word 3 for gfx9-family raw (untyped) buffers.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kAuxNT = 2;  // non-temporal: streamed weights are read once
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // a buffer offset the range check turns into zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ u32x4 load_beat(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxNT));
}

// Next work item for this wave: lane 0 takes a ticket from the workgroup's LDS counter.
__device__ __forceinline__ int claim_next(uint32_t *claim, int lane) {
    uint32_t v = 0;
    if (lane == 0) v = atomicAdd(claim, 1u);
    return (int)__builtin_amdgcn_readfirstlane(v);
}

// Bitwise select m ? p : n, written so the compiler emits one v_bitop3_b32.
__device__ __forceinline__ uint32_t select_bits(uint32_t m, uint32_t p, uint32_t n) { return ((p ^ n) & m) ^ n; }

// Sum over the 2^glog consecutive lanes of a row group; every lane of the group gets the total.
// Within 16 lanes DPP: swap pairs, swap halves of a quad, mirror within 8, mirror within 16.
__device__ __forceinline__ int32_t group_sum(int32_t s, int glog) {
    if (glog >= 1) s += __builtin_amdgcn_update_dpp(0, s, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    if (glog >= 2) s += __builtin_amdgcn_update_dpp(0, s, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    if (glog >= 3) s += __builtin_amdgcn_update_dpp(0, s, 0x141, 0xF, 0xF, false);  // row_half_mirror
    if (glog >= 4) s += __builtin_amdgcn_update_dpp(0, s, 0x140, 0xF, 0xF, false);  // row_mirror
    if (glog >= 5) s += __shfl_xor(s, 16);
    if (glog >= 6) s += __shfl_xor(s, 32);
    return s;
}

__device__ __forceinline__ void write_row(const DevJob &J, float x_scale, int row, int32_t s) {
    J.out_i32[row] = s;
    if (J.out_f32) {
        float t = (float)s * x_scale;   // exact integer (|s| < 2^24) times the activation scale
        J.out_f32[row] = t * J.w_scale;  // then the weight scale, each product rounded on its own
    }
}

// The job's activation scale: from device memory when the job names a location, else the table.
__device__ __forceinline__ float job_x_scale(const DevJob &J) { return J.x_scale_ptr ? *J.x_scale_ptr : J.x_scale; }

// ------------------------------------------------------------------------------------------
// Activation bit planes. Block b of x (64 int8 codes) becomes 16 words: word 2j + h holds bit j of
// columns 32h .. 32h+31, column 32h + k at bit k. In LDS, block b's four 16-byte quarters are
// rotated by (b >> 1) & 3, so the G blocks one wave reads at a time spread over all banks.

__device__ __forceinline__ int xq_slot(int b, int i) { return b * 4 + ((i + (b >> 1)) & 3); }

// Exchange of the bit fields selected by m (in x = hi:lo) with the fields S bits above them
// (a "delta swap"): t = (x ^ (x >> S)) & m; x ^= t ^ (t << S). Written on 32-bit halves; the 64-bit
// shifts of the halves become funnel shifts.
template <int S>
__device__ __host__ __forceinline__ void delta_swap(uint32_t &lo, uint32_t &hi, uint32_t mlo, uint32_t mhi) {
    const uint64_t x = ((uint64_t)hi << 32) | lo;
    const uint32_t tlo = (lo ^ (uint32_t)(x >> S)) & mlo;
    const uint32_t thi = (hi ^ (hi >> S)) & mhi;
    const uint64_t t = ((uint64_t)thi << 32) | tlo;
    lo ^= tlo ^ (tlo << S);
    hi ^= thi ^ (uint32_t)(t >> (32 - S));
}

// 8 x 8 bit-matrix transpose of the eight bytes in hi:lo (byte i = row i, bit j = column j): after
// it, byte j holds bit j of every input byte, input byte i at bit i. Three delta swaps at distances
// 7, 14 and 28 exchange the off-diagonal 1x1, 2x2 and 4x4 blocks: the published 8 x 8 transpose of
// H. S. Warren, "Hacker's Delight", section 7-3 ("Transposing a Bit Matrix"), with its masks.
__device__ __host__ __forceinline__ void transpose8x8(uint32_t &lo, uint32_t &hi) {
    delta_swap<7>(lo, hi, 0x00AA00AAu, 0x00AA00AAu);
    delta_swap<14>(lo, hi, 0x0000CCCCu, 0x0000CCCCu);
    delta_swap<28>(lo, hi, 0xF0F0F0F0u, 0u);
}

// Bit planes of one 16-byte piece of x (16 consecutive int8 codes, little-endian in w0..w3):
// plane[j] bit k = bit j of code k (j = 7 is the two's-complement sign bit).
__device__ __host__ __forceinline__ void piece_planes(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                                      uint32_t (&plane)[8]) {
    transpose8x8(w0, w1);  // codes 0..7
    transpose8x8(w2, w3);  // codes 8..15
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t a = j < 4 ? w0 : w1, b = j < 4 ? w2 : w3;
        const int sh = 8 * (j & 3);
        plane[j] = ((a >> sh) & 0xFFu) | (((b >> sh) & 0xFFu) << 8);
    }
}

// ------------------------------------------------------------------------------------------
// Select-accumulate core shared by the batch-1 and small-batch kernels. A row is served by
// G = 2^glog consecutive lanes; lane g holds beats g, g+G, ... of its row and reads the activation
// planes of those blocks from LDS (kXPassBlocks blocks, rotated as xq_slot says).

// Beats b = bbase + k*G of one row: zeros past bpr, past the matrix, or for a row-group that does
// not exist (live == false), all through offsets the buffer range check turns into zeros. The loads
// are issued on every path, so the compiler can count them and wait for exactly the older ones.
// NB > 0 is bpr known at compile time, which removes the bound checks that cannot fail.
template <int K, int NB>
__device__ __forceinline__ void issue_row(u32x4 (&B)[K], __amdgpu_buffer_rsrc_t wr, uint32_t row, bool live, int bbase,
                                          int G, int bpr) {
    const uint32_t rowoff = row * (uint32_t)bpr;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int b = bbase + k * G;
        const bool in = NB > 0 ? (b < NB) : (b < bpr);
        const uint32_t off = (live && in) ? (rowoff + (uint32_t)b) * 16u : kOutOfRange;
        B[k] = load_beat(wr, off);
    }
}

// The 16 plane words of block g + k*G (the block beat k of lane g covers). The index stays below
// K * G <= kXPassBlocks, inside the LDS copy, even past the pass or past bpr: there the beat is zero
// and the select yields zero whatever the words hold. When G is a multiple of 8 every block a lane
// reads has the rotation of block g, so the addresses are one base plus constant offsets.
template <int GLOG>
__device__ __forceinline__ void read_planes(uint32_t (&X)[16], const u32x4 *xl, int k, int g, int G) {
    const int b = g + k * G;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4 w = GLOG >= 3 ? xl[g * 4 + k * (4 << GLOG) + ((i + (g >> 1)) & 3)] : xl[xq_slot(b, i)];
        X[4 * i + 0] = w.x;
        X[4 * i + 1] = w.y;
        X[4 * i + 2] = w.z;
        X[4 * i + 3] = w.w;
    }
}

// acc += popc(v) as one accumulating v_bcnt_u32_b32. Written as an asm statement because with two
// popcounts into one counter the compiler emits two plain popcounts and a v_add3 instead (8 more VALU
// per beat; measured on the decode step: 77.2 against 77.9-78.1 us).
__device__ __forceinline__ void bcnt_acc(uint32_t &acc, uint32_t v) {
    asm("v_bcnt_u32_b32 %0, %1, %0" : "+v"(acc) : "v"(v));
}

// Exact partial sum of one row over the K beats a lane holds, activation planes from LDS:
//   sum_j w_j * popc(select(X_j, pos, neg)) + popc(neg),  w_j = 2^j, w_7 = -128.
// The planes of beat k+1 are read while beat k is reduced; the empty asm statements keep the
// compiler from hoisting every beat's reads (16 registers per beat, and the occupancy this kernel
// relies on).
template <int K, int GLOG>
__device__ __forceinline__ int32_t row_partial(const u32x4 *xl, const u32x4 (&B)[K], int g, int G) {
    uint32_t c[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    uint32_t cn = 0;
    uint32_t Xa[16], Xb[16];
    read_planes<GLOG>(Xa, xl, 0, g, G);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        uint32_t(&X)[16] = (k & 1) ? Xb : Xa;
        uint32_t(&Xn)[16] = (k & 1) ? Xa : Xb;
        if (k + 1 < K) read_planes<GLOG>(Xn, xl, k + 1, g, G);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            c[j] = __builtin_popcount(select_bits(X[2 * j], B[k].x, B[k].z)) + c[j];
            bcnt_acc(c[j], select_bits(X[2 * j + 1], B[k].y, B[k].w));
        }
        cn = __builtin_popcount(B[k].z) + cn;
        cn = __builtin_popcount(B[k].w) + cn;
        asm volatile("" : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]), "+v"(c[4]), "+v"(c[5]), "+v"(c[6]),
                     "+v"(c[7]), "+v"(cn)::"memory");
    }
    int32_t acc = (int32_t)cn;
#pragma unroll
    for (int j = 0; j < 7; ++j) acc += (int32_t)(c[j] << j);
    acc -= (int32_t)(c[7] << 7);
    return acc;
}

// Planes of blocks [b0, b0 + nb) of x (nb <= kXPassBlocks), built in LDS by the workgroup's waves
// in turn, 16 blocks per wave-round: a lane loads one 16-byte piece (piece p = block p / 4, quarter
// p % 4) and stores its 16 bits of every plane as one 16-bit LDS write. Pieces of the last round
// past nb * 4 read zeros through the buffer range check and write zero planes into blocks no beat
// of this pass selects from. Each trip consumes its own load, so no load is left outstanding behind
// the (wave-uniform) loop.
__device__ __forceinline__ void stage_planes(u32x4 *xl, const int8_t *x, int b0, int nb, int wave, int lane) {
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (int64_t)b0 * 64, (uint32_t)nb * 64u);
    const int need = (nb * 4 + 63) / 64;  // waves' worth of pieces
    uint16_t *xh = reinterpret_cast<uint16_t *>(xl);
    for (int wv = wave; wv < need; wv += kWaves) {
        const int p = wv * 64 + lane;
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)p * 16u, 0, 0));
        const int b = p >> 2, qq = p & 3;
        uint32_t pl[8];
        piece_planes(v.x, v.y, v.z, v.w, pl);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int w = 2 * j + (qq >> 1);
            xh[(xq_slot(b, w >> 2) * 4 + (w & 3)) * 2 + (qq & 1)] = (uint16_t)pl[j];
        }
    }
}

// ------------------------------------------------------------------------------------------
// Byte-lane select ("The .trit format, version 1", section 1: the masks pick the activation bytes that
// are added and subtracted). Each 4-bit group of a mask is widened to four byte lanes
// (n * 0x00204081 puts bit i at bit 7i; & 0x01010101 keeps bits 0, 8, 16 and 24) and a signed 4-way
// int8 dot product (v_dot4_i32_i8) adds the selected bytes of x.

__device__ __forceinline__ int32_t spread4(uint32_t m, int i) {
    return (int32_t)((((m >> (4 * i)) & 0xFu) * 0x00204081u) & 0x01010101u);
}

// Blocks [b0, b0 + nb) of x as they are (16 words of four int8 codes per block, word w = columns
// 4w .. 4w+3), in the LDS slots the bit planes use (xq_slot), one 16-byte piece per lane; the same
// zero-filled last round as stage_planes.
__device__ __forceinline__ void stage_bytes(u32x4 *xl, const int8_t *x, int b0, int nb, int wave, int lane) {
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x + (int64_t)b0 * 64, (uint32_t)nb * 64u);
    const int need = (nb * 4 + 63) / 64;
    for (int wv = wave; wv < need; wv += kWaves) {
        const int p = wv * 64 + lane;
        xl[xq_slot(p >> 2, p & 3)] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)p * 16u, 0, 0));
    }
}

// Exact partial sum of one row over the K beats a lane holds, activation bytes from LDS: the +1 lanes'
// dot product minus the -1 lanes'. Same read-ahead and scheduling barrier as row_partial.
template <int K, int GLOG>
__device__ __forceinline__ int32_t row_partial_bytelane(const u32x4 *xl, const u32x4 (&B)[K], int g, int G) {
    int32_t ap = 0, an = 0;
    uint32_t Xa[16], Xb[16];
    read_planes<GLOG>(Xa, xl, 0, g, G);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        uint32_t(&X)[16] = (k & 1) ? Xb : Xa;
        uint32_t(&Xn)[16] = (k & 1) ? Xa : Xb;
        if (k + 1 < K) read_planes<GLOG>(Xn, xl, k + 1, g, G);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ap = __builtin_amdgcn_sdot4(spread4(B[k].x, i), (int32_t)X[i], ap, false);
            an = __builtin_amdgcn_sdot4(spread4(B[k].z, i), (int32_t)X[i], an, false);
            ap = __builtin_amdgcn_sdot4(spread4(B[k].y, i), (int32_t)X[8 + i], ap, false);
            an = __builtin_amdgcn_sdot4(spread4(B[k].w, i), (int32_t)X[8 + i], an, false);
        }
        asm volatile("" : "+v"(ap), "+v"(an)::"memory");
    }
    return ap - an;
}

static inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace bpw

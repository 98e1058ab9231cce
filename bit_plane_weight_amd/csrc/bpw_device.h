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

__device__ __forceinline__ void write_row(const DevJob &J, int row, int32_t s) {
    J.out_i32[row] = s;
    if (J.out_f32) {
        float t = (float)s * J.x_scale;  // exact integer (|s| < 2^24) times the activation scale
        J.out_f32[row] = t * J.w_scale;  // then the weight scale, each product rounded on its own
    }
}

// ------------------------------------------------------------------------------------------
// Activation bit planes. Block b of x (64 int8 codes) becomes 16 words: word 2j + h holds bit j of
// columns 32h .. 32h+31, column 32h + k at bit k. In LDS, block b's four 16-byte quarters are
// rotated by (b >> 1) & 3, so the G blocks one wave reads at a time spread over all banks.

__device__ __forceinline__ int xq_slot(int b, int i) { return b * 4 + ((i + (b >> 1)) & 3); }

// Bit j of each byte of d, gathered into bits 0..3 (byte i -> bit i). After the mask the four bits
// sit at 0, 8, 16 and 24; multiplying by 2^24 + 2^17 + 2^10 + 2^3 lands them on 24..27, and no two
// of the sixteen shifted copies share a bit position, so nothing carries into that field.
__device__ __forceinline__ uint32_t byte_bits(uint32_t d, int j) {
    return (((d >> j) & 0x01010101u) * 0x01020408u) >> 24;
}

// Planes of one 16-column piece of x (the 16 bytes in v) for bit j: column k of the piece at bit k.
__device__ __forceinline__ uint32_t piece_plane(const u32x4 &v, int j) {
    return byte_bits(v.x, j) | (byte_bits(v.y, j) << 4) | (byte_bits(v.z, j) << 8) | (byte_bits(v.w, j) << 12);
}

static inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace bpw

// bpw_bitcos.hip - batch-1 grouped GEMV on BITCOS matrices for gfx950.
//
// BITCOS ("BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits", "A bitmap and a sign")
// stores a presence bit per weight and a sign bit per nonzero, compacted in column order. The kernel
// turns each 64-column block back into the pos/neg planes of the .trit beat and then runs the same
// bit-serial select-accumulate as the .trit kernel. Decoding a block is a bit deposit: the block's
// sign bits go, in order, to the set positions of its presence word (neg); pos = presence & ~neg.
// gfx950 has no deposit instruction, so it is done a byte at a time through a 64 KiB LDS table
// (presence byte | eight sign bits -> neg byte; the page's GPU decoder uses a 256-entry table on
// nibbles, which costs twice the lookups and index arithmetic here).
//
// Lane layout: the G lanes of a row (8, 16 or 32, by row width) hold contiguous runs of K blocks
// (lane g: blocks gK .. gK+K-1), so a row needs one prefix sum of the lanes' nonzero counts to place
// every lane's signs; within a lane the offset of block k is a running sum. The activation planes are
// staged in LDS in the order the lanes read them (slot k*G + g). Each wave keeps the loads of its next
// two row-groups in flight while it decodes one. Launched only by bpw_bitcos_host.cpp after its
// argument and architecture checks.
#include <hip/hip_runtime.h>

#include "bpw_device.h"

namespace bpw {

namespace {

struct Deposit8Table {
    uint8_t v[65536];
};

// Four-bit deposit: the low bits of s, in order, into the set positions of p.
constexpr uint8_t deposit4(uint32_t p, uint32_t s) {
    uint32_t out = 0, k = 0;
    for (int b = 0; b < 4; ++b)
        if ((p >> b) & 1u) {
            out |= ((s >> k) & 1u) << b;
            ++k;
        }
    return (uint8_t)out;
}

// Entry p | s << 8: the low popc(p) bits of s deposited into the set positions of the byte p (two
// nibble deposits, the high nibble's signs starting after the low nibble's).
constexpr Deposit8Table make_deposit8() {
    Deposit8Table t{};
    uint8_t d4[256] = {};  // d4[p | s << 4] = deposit4(p, s)
    for (uint32_t i = 0; i < 256; ++i) d4[i] = deposit4(i & 15u, i >> 4);
    for (uint32_t i = 0; i < 65536; ++i) {
        const uint32_t p = i & 255u, s = i >> 8, lo = p & 15u;
        const uint32_t c = (lo & 1u) + ((lo >> 1) & 1u) + ((lo >> 2) & 1u) + ((lo >> 3) & 1u);
        t.v[i] = (uint8_t)(d4[lo | ((s & 15u) << 4)] | (d4[(p >> 4) | (((s >> c) & 15u) << 4)] << 4));
    }
    return t;
}

}  // namespace

__device__ constexpr Deposit8Table kDeposit8 = make_deposit8();

// LDS of one workgroup: the activation planes, one slot of kBcSlotQuarters 16-byte quarters per
// block (four used), then the deposit table. The odd slot stride puts the G blocks one instruction
// reads (consecutive slots) in distinct bank groups, 16 lanes at a time. Both arrays start below
// 64 KiB, so every plane read and table lookup takes its array's address as the instruction's
// immediate offset.
constexpr int kBcSlotQuarters = 5;
struct BcShared {
    u32x4 xl[kXPassBlocks * kBcSlotQuarters];
    uint8_t lut[65536];
};

// The sign bits of a 32-bit presence word p, s holding them from bit 0: neg = deposit(s, p).
// Byte t's signs start after the nonzeros of the bytes below it; v_perm builds each table index
// (presence byte t | the byte of s at that offset << 8) in one instruction.
__device__ __forceinline__ uint32_t deposit32(const uint8_t *lut, uint32_t p, uint32_t s) {
    const uint32_t r1 = __builtin_popcount(p & 0xFFu);
    const uint32_t r2 = __builtin_popcount(p & 0xFFFFu);
    const uint32_t r3 = __builtin_popcount(p & 0xFFFFFFu);
    const uint32_t i0 = __builtin_amdgcn_perm(s, p, 0x0C0C0400u);
    const uint32_t i1 = __builtin_amdgcn_perm(s >> r1, p, 0x0C0C0401u);
    const uint32_t i2 = __builtin_amdgcn_perm(s >> r2, p, 0x0C0C0402u);
    const uint32_t i3 = __builtin_amdgcn_perm(s >> r3, p, 0x0C0C0403u);
    const uint32_t n01 = __builtin_amdgcn_perm((uint32_t)lut[i1], (uint32_t)lut[i0], 0x0C0C0400u);
    const uint32_t n23 = __builtin_amdgcn_perm((uint32_t)lut[i3], (uint32_t)lut[i2], 0x0C0C0400u);
    return n01 | (n23 << 16);
}

// Exclusive sum over the lanes g' < g of an aligned group of G = 2^GLOG lanes. DPP row shifts give
// lanes whose source lies before their 16-lane row a zero; groups of 8 also drop sources from the
// other half of the row, and groups of 32 add the last lane of the row below (row_bcast:15).
template <int GLOG>
__device__ __forceinline__ uint32_t exclusive_scan(uint32_t v, int g) {
    const uint32_t v0 = v;
    uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += (GLOG > 3 || g >= 1) ? t : 0u;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += (GLOG > 3 || g >= 2) ? t : 0u;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += (GLOG > 3 || g >= 4) ? t : 0u;
    if constexpr (GLOG >= 4) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    if constexpr (GLOG >= 5) v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    static_assert(GLOG >= 3 && GLOG <= 5, "8, 16 or 32 lanes per row");
    return v - v0;
}

// Where lane g's k-th block (block gK + k of the row) sits in the staged planes: slot k * G + g, so
// the G blocks one instruction reads are consecutive slots.
__device__ __forceinline__ int bc_quarter(int k, int g, int G, int i) { return (k * G + g) * kBcSlotQuarters + i; }

// Planes of blocks [0, nb) of x into LDS in the slot order above (the bit transposition of
// stage_planes; one 16-byte piece of x per lane, a 16-bit store per plane). Blocks past K * G are
// never read and not stored.
__device__ __forceinline__ void bc_stage(u32x4 *xl, const int8_t *x, int nb, int K, int G, int wave, int lane) {
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)nb * 64u);
    const int need = (nb * 4 + 63) / 64;
    uint16_t *xh = reinterpret_cast<uint16_t *>(xl);
    for (int wv = wave; wv < need; wv += kBcWaves) {
        const int p = wv * 64 + lane;
        const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)p * 16u, 0, 0));
        const int b = p >> 2, qq = p & 3;
        uint32_t pl[8];
        piece_planes(v.x, v.y, v.z, v.w, pl);
        if (b < K * G) {
            const int g = b / K, k = b - g * K;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int w = 2 * j + (qq >> 1);
                xh[(bc_quarter(k, g, G, w >> 2) * 4 + (w & 3)) * 2 + (qq & 1)] = (uint16_t)pl[j];
            }
        }
    }
}

// A row's presence words as lane g holds them (blocks gK .. gK+K-1; zeros past bpr, past the
// matrix, or for a row-group that does not exist) and the row's first sign word.
template <int K>
struct BcPresence {
    uint32_t lo[K], hi[K];
    uint32_t rs;
};

struct BcRowCtx {
    __amdgpu_buffer_rsrc_t pr, rr, sr;
    int bpr, rows, g;
};

// Cached loads: one instruction reads every K-th word of the row, so the row's lines serve K
// instructions in turn (non-temporal loads refetched them: 16 % more HBM traffic, 18 % slower).
template <int K>
__device__ __forceinline__ void bc_load_presence(BcPresence<K> &P, const BcRowCtx &c, int row, bool live) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int b = c.g * K + k;
        const uint32_t off = (live && b < c.bpr) ? ((uint32_t)row * (uint32_t)c.bpr + (uint32_t)b) * 8u : kOutOfRange;
        const uint64_t v = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(c.pr, off, 0, 0));
        P.lo[k] = (uint32_t)v;
        P.hi[k] = (uint32_t)(v >> 32);
    }
    P.rs = __builtin_amdgcn_raw_buffer_load_b32(c.rr, live ? (uint32_t)row * 4u : kOutOfRange, 0, 0);
}

// Sign windows of the lane's K blocks: 96 bits of the row's sign words from the word holding the
// block's first sign (none for a block without nonzeros); .w keeps the bit offset in that word. The
// lane's first sign index is the prefix sum of the row's lanes' nonzero counts.
template <int K, int GLOG>
__device__ __forceinline__ void bc_load_windows(u32x4 (&W)[K], const BcPresence<K> &P, const BcRowCtx &c, bool live) {
    uint32_t n = 0;
#pragma unroll
    for (int k = 0; k < K; ++k) n = __builtin_popcount(P.hi[k]) + (__builtin_popcount(P.lo[k]) + n);
    uint32_t o = exclusive_scan<GLOG>(n, c.g);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint32_t nk = __builtin_popcount(P.lo[k]) + __builtin_popcount(P.hi[k]);
        const uint32_t off = (live && nk != 0) ? (P.rs + (o >> 5)) * 4u : kOutOfRange;
        W[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c.sr, off, 0, 0));
        W[k].w = o & 31u;
        o += nk;
    }
}

// Decode the lane's K blocks to planes and accumulate their select-popcounts (cs[j], ch[j]: plane j
// over the low and high 32 columns; cn: neg).
template <int K, int GLOG>
__device__ __forceinline__ void bc_decode(uint32_t (&cs)[8], uint32_t (&ch)[8], uint32_t &cn, const BcPresence<K> &P,
                                          const u32x4 (&W)[K], const BcShared &sh, const BcRowCtx &c) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint32_t p0 = P.lo[k], p1 = P.hi[k];
        const uint32_t shf = W[k].w;
        const uint32_t s_lo = __builtin_amdgcn_alignbit(W[k].y, W[k].x, shf);
        const uint32_t s_hi = __builtin_amdgcn_alignbit(W[k].z, W[k].y, shf);
        const uint32_t pcl = __builtin_popcount(p0);
        const uint32_t s2 = pcl == 32u ? s_hi : __builtin_amdgcn_alignbit(s_hi, s_lo, pcl);
        const uint32_t nlo = deposit32(sh.lut, p0, s_lo);
        const uint32_t nhi = deposit32(sh.lut, p1, s2);
        const uint32_t qlo = p0 & ~nlo, qhi = p1 & ~nhi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 X = sh.xl[bc_quarter(k, c.g, 1 << GLOG, i)];
            // words 4i .. 4i+3: planes 2i (lo, hi) and 2i + 1 (lo, hi); the halves count separately, so
            // each popcount adds into its own counter in one v_bcnt_u32_b32
            cs[2 * i] = __builtin_popcount(select_bits(X.x, qlo, nlo)) + cs[2 * i];
            ch[2 * i] = __builtin_popcount(select_bits(X.y, qhi, nhi)) + ch[2 * i];
            cs[2 * i + 1] = __builtin_popcount(select_bits(X.z, qlo, nlo)) + cs[2 * i + 1];
            ch[2 * i + 1] = __builtin_popcount(select_bits(X.w, qhi, nhi)) + ch[2 * i + 1];
        }
        cn = __builtin_popcount(nlo) + cn;
        cn = __builtin_popcount(nhi) + cn;
        // keep the next block's table and plane reads (and any later load) below this block: hoisted,
        // they would hold more registers than the occupancy allows
        asm volatile("" : "+v"(cs[0]), "+v"(cs[1]), "+v"(cs[2]), "+v"(cs[3]), "+v"(cs[4]), "+v"(cs[5]), "+v"(cs[6]),
                     "+v"(cs[7]), "+v"(ch[0]), "+v"(ch[1]), "+v"(ch[2]), "+v"(ch[3]), "+v"(ch[4]), "+v"(ch[5]),
                     "+v"(ch[6]), "+v"(ch[7]), "+v"(cn)::"memory");
    }
}

// Rows of the tile's row-groups [u0, u1): wave w takes row-groups u0 + w, u0 + w + kBcWaves, ...
// (at most kIt of them), lane g of row q = lane / G holding blocks gK .. gK+K-1. Loads run ahead of
// the decode: iteration i issues the presence loads of row-group i, the sign loads of row-group
// i - 1 (its presence has arrived) and decodes row-group i - 2 (its signs have arrived). Row-groups
// past the tile load zeros through the range check and write nothing.
template <int K, int GLOG>
__device__ __forceinline__ void bc_tile(const BitcosJob &J, int u0, int u1, int wave, int lane, const BcShared &sh,
                                        const BcRowCtx &c) {
    constexpr int kIt = kBcTileUnits / kBcWaves;
    constexpr int kUnitRows = 64 >> GLOG;
    const int q = lane >> GLOG;
    BcPresence<K> P[kIt];
    u32x4 W[kIt][K];
#pragma unroll
    for (int i = 0; i < kIt + 2; ++i) {
        if (i < kIt) {
            const int u = u0 + wave + i * kBcWaves, row = u * kUnitRows + q;
            bc_load_presence(P[i], c, row, u < u1 && row < J.rows);
        }
        if (i >= 1 && i - 1 < kIt) {
            const int u = u0 + wave + (i - 1) * kBcWaves, row = u * kUnitRows + q;
            bc_load_windows<K, GLOG>(W[i - 1], P[i - 1], c, u < u1 && row < J.rows);
        }
        const int ud = u0 + wave + (i - 2) * kBcWaves;
        if (i >= 2 && ud < u1) {  // wave-uniform
            const int row = ud * kUnitRows + q;
            uint32_t cs[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
            uint32_t ch[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
            uint32_t cn = 0;
            bc_decode<K, GLOG>(cs, ch, cn, P[i - 2], W[i - 2], sh, c);
            int32_t acc = (int32_t)cn;
#pragma unroll
            for (int j = 0; j < 7; ++j) acc += (int32_t)((cs[j] + ch[j]) << j);
            acc -= (int32_t)((cs[7] + ch[7]) << 7);
            const int32_t tot = group_sum(acc, GLOG);
            if (c.g == 0 && row < J.rows) {
                J.out_i32[row] = tot;
                if (J.out_f32) J.out_f32[row] = ((float)tot * J.x_scale) * J.w_scale;  // the scales in turn
            }
        }
    }
}

__global__ __launch_bounds__(kBcThreads, 4) void gemv_bitcos_kernel(const BitcosJob *__restrict__ jobs,
                                                                     const Tile *__restrict__ tiles) {
    __shared__ BcShared sh;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const Tile t = tiles[blockIdx.x];
    const BitcosJob J = jobs[t.job];
    const BcGeometry geo = bitcos_geometry(J.bpr);
    {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(kDeposit8.v);
        u32x4 *dst = reinterpret_cast<u32x4 *>(sh.lut);
#pragma unroll
        for (int i = 0; i < 65536 / 16 / kBcThreads; ++i) dst[i * kBcThreads + threadIdx.x] = src[i * kBcThreads + threadIdx.x];
    }
    bc_stage(sh.xl, J.x, J.bpr, geo.k, 1 << geo.glog, wave, lane);
    __syncthreads();
    BcRowCtx c;
    c.pr = make_rsrc(J.presence, J.presence_bytes);
    c.rr = make_rsrc(J.row_start, J.row_start_bytes);
    c.sr = make_rsrc(J.signs, J.sign_bytes);
    c.bpr = J.bpr;
    c.rows = J.rows;
    c.g = lane & ((1 << geo.glog) - 1);
    if (geo.glog == 3 && geo.k == 2)
        bc_tile<2, 3>(J, t.u0, t.u1, wave, lane, sh, c);
    else if (geo.glog == 3)
        bc_tile<5, 3>(J, t.u0, t.u1, wave, lane, sh, c);
    else if (geo.glog == 4)
        bc_tile<4, 4>(J, t.u0, t.u1, wave, lane, sh, c);
    else
        bc_tile<4, 5>(J, t.u0, t.u1, wave, lane, sh, c);
}

int launch_gemv_bitcos(const BitcosJob *jobs, const Tile *tiles, int32_t n_tiles, void *stream) {
    if (n_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(gemv_bitcos_kernel, dim3((unsigned)n_tiles), dim3(kBcThreads), 0, as_stream(stream), jobs, tiles);
    return hipGetLastError();
}

}  // namespace bpw

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
// Small batch on the matrix cores: v_mfma_i32_16x16x64_i8 multiplies 16 rows x 64 columns of int8
// weights by 64 columns x 16 tokens of int8 activations into 16 x 16 int32 sums. The planes are
// decoded to int8 weights once per beat, whatever the batch. Decoding goes through a 256-entry LDS
// table: entry (p | n << 4) holds the four weights of a nibble pair of the planes (byte k = +1 if
// bit k of p, -1 if bit k of n, else 0; P1 rules out both).
//
// A workgroup owns 16 rows x up to 16 tokens; its waves (4, or 8 for rows of more than 64 blocks)
// split the row's beats (iteration i covers blocks 4i .. 4i+3, wave w takes i = w, w + waves, ...),
// and the partial sums meet in LDS. In one iteration lane l holds the beat of row l % 16, block 4i + l / 16, and for each
// quarter m of that block the 16 activation bytes of token l % 16 at the same columns: the
// instruction pairs byte j of lane l's weights with byte j of the activations of lanes with the
// same l / 16, so both operands only have to agree on the column order, which they do. Result lane
// l, register r holds row 4 * (l / 16) + r, token l % 16.

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaRows = 16;    // rows per workgroup
constexpr int kMfmaTokens = 16;  // tokens per workgroup

__device__ __forceinline__ uint32_t lut_entry(uint32_t idx) {
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if ((idx >> k) & 1u)
            w |= 0x01u << (8 * k);
        else if ((idx >> (4 + k)) & 1u)
            w |= 0xFFu << (8 * k);
    }
    return w;
}

// Weights of columns 16m .. 16m+15 of a beat as the 16 int8 bytes of one operand. e and o hold the
// table indices of the even and odd nibbles of the beat's 32-bit half that contains them.
__device__ __forceinline__ v4i decode_quarter(const uint32_t *lut, uint32_t e, uint32_t o, int m) {
    const int sh = 16 * (m & 1);
    v4i a;
    a.x = (int)lut[(e >> sh) & 0xFFu];        // columns 16m + 0..3
    a.y = (int)lut[(o >> sh) & 0xFFu];        // 4..7
    a.z = (int)lut[(e >> (sh + 8)) & 0xFFu];  // 8..11
    a.w = (int)lut[(o >> (sh + 8)) & 0xFFu];  // 12..15
    return a;
}

// Loads of one iteration: the beat of (row, block b) and the four 16-byte activation pieces of
// token tok at block b. Past the matrix, past bpr or past the batch they read zeros through the
// buffer range checks; they are issued on every path so the compiler counts them exactly.
__device__ __forceinline__ void mfma_issue(u32x4 &beat, u32x4 (&xv)[4], __amdgpu_buffer_rsrc_t wr,
                                           __amdgpu_buffer_rsrc_t xr, uint32_t row, uint32_t tok, int b, int bpr,
                                           int64_t ldx, bool live) {
    const bool in = live && b < bpr;
    beat = load_beat(wr, in ? (row * (uint32_t)bpr + (uint32_t)b) * 16u : kOutOfRange);
    const uint32_t xo = (uint32_t)((int64_t)tok * ldx + (int64_t)b * 64);
#pragma unroll
    for (int m = 0; m < 4; ++m)
        xv[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, in ? xo + 16u * m : kOutOfRange, 0, 0));
}

// One iteration's four products: the beat's nibble-pair table indices (e: even nibbles, o: odd
// nibbles of each 32-bit half, byte k = p nibble | n nibble << 4), then one instruction per quarter.
__device__ __forceinline__ v4i mfma_beat(const uint32_t *lut, const u32x4 &beat, const u32x4 (&xv)[4], v4i acc) {
    const uint32_t elo = (beat.x & 0x0F0F0F0Fu) | ((beat.z << 4) & 0xF0F0F0F0u);
    const uint32_t olo = ((beat.x >> 4) & 0x0F0F0F0Fu) | (beat.z & 0xF0F0F0F0u);
    const uint32_t ehi = (beat.y & 0x0F0F0F0Fu) | ((beat.w << 4) & 0xF0F0F0F0u);
    const uint32_t ohi = ((beat.y >> 4) & 0x0F0F0F0Fu) | (beat.w & 0xF0F0F0F0u);
#pragma unroll
    for (int m = 0; m < 4; ++m)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_quarter(lut, m < 2 ? elo : ehi, m < 2 ? olo : ohi, m),
                                                    __builtin_bit_cast(v4i, xv[m]), acc, 0, 0, 0);
    return acc;
}

// The decode table, filled by the first 256 threads of the workgroup (made visible by the barrier in
// mfma_tile).
__device__ __forceinline__ void fill_lut(uint32_t *lut) {
    if (threadIdx.x < 256) lut[threadIdx.x] = lut_entry(threadIdx.x);
}

// Rows 16 * row_tile .. +15 and tokens 16 * tok_group .. +15 of the call A, by the workgroup's WAVES
// waves. part holds one partial per wave and lane.
template <int WAVES>
__device__ __forceinline__ void mfma_tile(const SmallBatchArgs &A, uint32_t row_tile, uint32_t tok_group,
                                          const uint32_t *lut, v4i (*part)[64]) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t row = row_tile * kMfmaRows + (lane & 15);
    const uint32_t tok = tok_group * kMfmaTokens + (lane & 15);
    const int bq = lane >> 4;  // which block of the iteration's four this lane holds
    const int bpr = A.bpr;
    const int n_it = (bpr + 3) / 4;
    const int64_t ldx = A.ldx;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(A.planes, A.plane_bytes);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(A.X, A.x_bytes);
    __syncthreads();  // the table is complete
    v4i acc = {0, 0, 0, 0};
    u32x4 beat0, beat1, x0[4], x1[4];
    int it = wave;
    mfma_issue(beat0, x0, wr, xr, row, tok, 4 * it + bq, bpr, ldx, it < n_it);
    // Two load sets alternate, as in the batch-1 kernel: iteration it + WAVES is in flight while
    // iteration it is multiplied; one trip covers two iterations with no exit in between.
    for (; it < n_it; it += 2 * WAVES) {
        mfma_issue(beat1, x1, wr, xr, row, tok, 4 * (it + WAVES) + bq, bpr, ldx, it + WAVES < n_it);
        asm volatile("" ::: "memory");
        acc = mfma_beat(lut, beat0, x0, acc);
        mfma_issue(beat0, x0, wr, xr, row, tok, 4 * (it + 2 * WAVES) + bq, bpr, ldx, it + 2 * WAVES < n_it);
        asm volatile("" ::: "memory");
        acc = mfma_beat(lut, beat1, x1, acc);
    }
    part[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x >= 256) return;
    // thread t < 256 sums register t / 64 of lane t % 64 over the waves (exact) and stores it
    const int l = threadIdx.x & 63, r = threadIdx.x >> 6;
    int32_t sum = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += part[w][l][r];
    const int orow = (int)row_tile * kMfmaRows + 4 * (l >> 4) + r;
    const int otok = (int)tok_group * kMfmaTokens + (l & 15);
    if (orow < A.rows && otok < A.batch) {
        const int64_t idx = (int64_t)otok * A.rows + orow;
        A.out_i32[idx] = sum;
        if (A.out_f32) {
            const float f = (float)sum * A.x_scales[otok];  // exact integer times the token's scale
            A.out_f32[idx] = f * A.w_scale;                  // then the weight scale
        }
    }
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_small_batch_mfma_kernel(SmallBatchArgs A) {
    static_assert(64 * WAVES >= 256, "every thread of the first four waves fills one table entry");
    __shared__ uint32_t lut[256];
    __shared__ v4i part[WAVES][64];
    fill_lut(lut);
    mfma_tile<WAVES>(A, blockIdx.x, blockIdx.y, lut, part);
}

// A beat load without the non-temporal hint. One iteration reads 64 of the 128 bytes of a row's cache
// line and the next iteration the other 64; with the hint the fetch counter showed 1.68x the plane
// bytes read from HBM on the decode-step set, cached it shows 1.02x (batch 2).
__device__ __forceinline__ u32x4 load_beat_cached(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The decode table of the grouped launch in kLutCopies = 32 copies: entry e is a 256-byte LDS row whose
// first 128 bytes hold its copies (copy c at e * 256 + 4 c) and whose last 128 bytes hold activation
// operands (see op_base). Lane l reads copy l % 32, so the 32 lanes the LDS serves together hit 32
// different banks whatever entries they ask for (with one shared copy the random entries of a wave's
// lookups collided: 3.1 bank conflicts per lookup, measured).
constexpr int kLutCopies = 32;
constexpr int kLutRowBytes = 256;
constexpr int kLutBytes = 256 * kLutRowBytes;  // address span of the table; half of it is operands

__device__ __forceinline__ void fill_lut_copies(uint32_t *lut, int nthreads) {
    uint8_t *base = reinterpret_cast<uint8_t *>(lut);
    for (int i = (int)threadIdx.x; i < 256 * (kLutCopies / 4); i += nthreads) {
        const uint32_t v = lut_entry((uint32_t)i / (kLutCopies / 4));
        *reinterpret_cast<u32x4 *>(base + (i / (kLutCopies / 4)) * kLutRowBytes + (i % (kLutCopies / 4)) * 16) =
            u32x4{v, v, v, v};
    }
}

// This lane's constant part of a table address (see lut_addr).
__device__ __forceinline__ uint32_t lut_lane_bits(int lane) { return (uint32_t)(lane % kLutCopies) << 2; }

// LDS byte address of the entry named by byte k of w, in this lane's copy: e * 256 + 4 (lane % 32). One
// v_perm_b32 places byte k of w in byte 1 and the lane bits in byte 0 (selectors 4 + k and 0; 0x0C gives
// zero bytes 2 and 3), which is the address itself. Below kLutBytes for any input. (With the copies
// packed 128 bytes apart, each address needed a shift as well: 64 of a step's 201 VALU.)
__device__ __forceinline__ uint32_t lut_addr(uint32_t w, int k, uint32_t lane_bits) {
    return __builtin_amdgcn_perm(w, lane_bits, 0x0C0C0000u | ((4u + (uint32_t)k) << 8));
}

__device__ __forceinline__ int lut_at(const uint32_t *lut, uint32_t addr) {
    return (int)*reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(lut) + addr);
}

// As decode_quarter, through this lane's copy of the table.
__device__ __forceinline__ v4i decode_quarter_own(const uint32_t *lut, uint32_t e, uint32_t o, int m, uint32_t lb) {
    const int b = 2 * (m & 1);
    v4i a;
    a.x = lut_at(lut, lut_addr(e, b, lb));      // columns 16m + 0..3
    a.y = lut_at(lut, lut_addr(o, b, lb));      // 4..7
    a.z = lut_at(lut, lut_addr(e, b + 1, lb));  // 8..11
    a.w = lut_at(lut, lut_addr(o, b + 1, lb));  // 12..15
    return a;
}

__device__ __forceinline__ v4i mfma_beat_own(const uint32_t *lut, const u32x4 &beat, const u32x4 (&xv)[4], v4i acc,
                                             uint32_t lb) {
    const uint32_t elo = (beat.x & 0x0F0F0F0Fu) | ((beat.z << 4) & 0xF0F0F0F0u);
    const uint32_t olo = ((beat.x >> 4) & 0x0F0F0F0Fu) | (beat.z & 0xF0F0F0F0u);
    const uint32_t ehi = (beat.y & 0x0F0F0F0Fu) | ((beat.w << 4) & 0xF0F0F0F0u);
    const uint32_t ohi = ((beat.y >> 4) & 0x0F0F0F0Fu) | (beat.w & 0xF0F0F0F0u);
#pragma unroll
    for (int m = 0; m < 4; ++m)
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_quarter_own(lut, m < 2 ? elo : ehi, m < 2 ? olo : ohi, m, lb),
                                                    __builtin_bit_cast(v4i, xv[m]), acc, 0, 0, 0);
    return acc;
}

// The weight stream of a wave. The matrix cores want lane l = 16 g + m to hold the beat of row m of a
// 16-row tile at block 4 i + g in iteration i, so a load in that layout covers 16 rows x 64 bytes:
// half cache lines, which a plain streaming read of the same rows showed at 4.1-4.9 TB/s (measured,
// loads only) against 6.9 for whole lines. A step therefore covers 8 blocks (two iterations) of a
// tile with two loads per lane whose address sets are rows 0-7 and rows 8-15, each 8 rows x 128 bytes
// (whole lines, non-temporal: 6.5-6.7 TB/s measured, loads only):
//   load j (j = 0, 1), lane 16 g + m: row 8 j + m % 8, block g + 4 [m / 8 != j]
// so that, with lo = (m < 8), the beats of the two iterations are
//   iteration 2s:     lo ? R0 : R1                          (row m, block g)
//   iteration 2s + 1: the value of (lo ? R1 : R0) in lane l ^ 8 (row m, block 4 + g)
// one select per word, and one DPP rotate by 8 within each row of 16 lanes.
__device__ __forceinline__ uint32_t swap8(uint32_t v) { return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false); }

__device__ __forceinline__ u32x4 step_first(const u32x4 &r0, const u32x4 &r1, bool lo) { return lo ? r0 : r1; }

__device__ __forceinline__ u32x4 step_second(const u32x4 &r0, const u32x4 &r1, bool lo) {
    const u32x4 t = lo ? r1 : r0;
    return u32x4{swap8(t.x), swap8(t.y), swap8(t.z), swap8(t.w)};
}

// The activation operands of up to kXtPassSteps steps sit in LDS: the matrix-core operand of quarter q
// of iteration h of a step is, in lane l = 16 g + n, codes 16 q .. 16 q + 15 of block 4 h + g of the
// step (8 blocks) of token n of the workgroup's token group. Loading them from memory in that order
// instead, each step's eight operand loads went through the same address path as the weights: the
// texture address unit stayed 67-76 % busy (counters) while the weights moved at less than half the
// batch-1 rate. Operand j = 4 h + q of a step is 1 KiB, 16 bytes per lane, placed as eight 128-byte
// pieces 256 bytes apart:
//   op_base(ls) + 2048 j + lane_off(l, q),   lane_off(l, q) = 256 (l / 8) + 16 ((l ^ s) % 8),
//   s = q + 4 ((l / 16) % 2)
// so that steps 0-3 of a pass fill the free halves of the table's rows (op_base = 16 KiB ls + 128 in the
// table) and steps 4-5 the two halves of a 16 KiB region after it. Eight lanes read one 128-byte piece,
// in some order: each ds_read_b128 stays conflict-free. The swizzle s serves the staging writes, where
// consecutive threads hold the quarters q and block groups g = l / 16 of one token: without it the 16
// lanes that the LDS serves at once all wrote the same 16-byte bank slot (13 M conflict cycles per
// launch at 16 tokens).
constexpr int kXtPassSteps = 6;       // 48 KiB of operands per pass (16 token slots)
constexpr int kXtStepBytes = 8192;    // 2 iterations x 4 quarters x 64 lanes x 16 bytes
constexpr int kXtTableSteps = kLutBytes / 2 / kXtStepBytes;  // steps held in the table's free halves
constexpr int kXtPieceStride = 2048;  // between the operands of one step
static_assert(kXtTableSteps == 4 && kXtPassSteps - kXtTableSteps == 2, "two steps in the region after the table");

__device__ __forceinline__ uint32_t lane_off(int lane, int q) {
    return (uint32_t)(lane >> 3) * 256u + (uint32_t)((lane ^ (q | ((lane >> 2) & 4))) & 7) * 16u;
}

// The first operand's 128-byte piece of step ls (0 <= ls < kXtPassSteps) for lane 0.
__device__ __forceinline__ uint8_t *op_base(uint32_t *lut, uint8_t *xl2, int ls) {
    return ls < kXtTableSteps ? reinterpret_cast<uint8_t *>(lut) + 128 + ls * (kXtStepBytes * 2)
                              : xl2 + (ls - kXtTableSteps) * 128;
}

// LDS of the grouped launch: the table in a static array (its address is then known when the kernel
// is compiled and folds into each lookup's instruction offset; from dynamic LDS every lookup paid a
// v_add of the base, 64 VALU per step), then the last two steps of a pass in dynamic LDS.
constexpr size_t kSbGroupedLds = (size_t)(kXtPassSteps - kXtTableSteps) * kXtStepBytes;
static_assert(2 * ((size_t)kLutBytes + kSbGroupedLds) <= 160 * 1024, "two workgroups per compute unit");

// One pass of the call's activation operands (the steps s0 .. s0 + kXtPassSteps - 1), read from X
// itself by all threads of the workgroup. Piece c of the pass is token n = c / kPassPieces of the
// workgroup's token group and 16-byte piece k = c % kPassPieces of that token's columns in the pass
// (block 8 s0 + k / 4 of the row, codes 16 (k % 4) .. +15), so consecutive threads read consecutive
// 16 bytes of one token's row; the piece goes to operand j = 4 ((k / 16) % 2) + k % 4 of local step
// k / 32, lane 16 ((k / 4) % 4) + n. Rounds that hold only tokens past the batch are skipped: those
// lanes' operands keep whatever LDS held, and only their own output columns, never stored, depend on
// them. Pieces past the row's blocks or past the batch read zeros through the buffer range check.
// Every load of a round is issued before the first LDS write. (A separate launch that wrote the
// operands out in the matrix cores' order first cost 5.9-6.4 us per run on the decode-step set, and
// 10.7 MB of writes.)
constexpr int kPassPieces = kXtPassSteps * 8 * 4;  // 16-byte pieces of one token's columns in a pass

template <int NT>
__device__ __forceinline__ void stage_x(uint32_t *lut, uint8_t *xl2, const SmallBatchArgs &A, int tok0, int s0) {
    static_assert((kMfmaTokens * kPassPieces) % NT == 0, "whole rounds");
    constexpr int kRounds = kMfmaTokens * kPassPieces / NT;
    const int real = min(kMfmaTokens, A.batch - tok0) * kPassPieces;  // pieces of tokens inside the batch
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(A.X, A.x_bytes);
    u32x4 v[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        if (r * NT >= real) break;  // uniform over the workgroup
        const int c = r * NT + (int)threadIdx.x;
        const int n = c / kPassPieces, k = c - n * kPassPieces;
        const int b = 8 * s0 + (k >> 2);
        const bool in = c < real && b < A.bpr;
        const uint32_t off = (uint32_t)((int64_t)(tok0 + n) * A.ldx + 64 * b + 16 * (k & 3));
        v[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, in ? off : kOutOfRange, 0, 0));
    }
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        if (r * NT >= real) break;
        const int c = r * NT + (int)threadIdx.x;
        const int n = c / kPassPieces, k = c - n * kPassPieces;
        const int bl = k >> 2;  // block within the pass
        *reinterpret_cast<u32x4 *>(op_base(lut, xl2, bl >> 3) + (4 * ((bl >> 2) & 1) + (k & 3)) * kXtPieceStride +
                                   lane_off(16 * (bl & 3) + n, k & 3)) = v[r];
    }
}

// Several calls in one launch. Workgroup b runs tile tiles[b]: kSBGroupRows rows x up to 16 tokens of
// one call. Each wave owns RT row tiles of 16 rows over every block of the row (no split of the row
// across waves); results leave straight from the matrix-core registers. The workgroup first stages
// the table and the call's activation operands in LDS; rows wider than kXtPassSteps steps take several
// passes, the operands of each staged in turn (every wave, with rows or not, takes part in the staging).
// Within a pass the beats of the next ST - 1 steps are in flight while a step is decoded and multiplied
// (ST register sets, the step loop unrolled ST times so each set is fixed; a wave with few waves per
// compute unit needs several steps of weights in flight to cover the memory latency under load); the
// first ST - 1 steps' beats leave before the pass's operands are staged. Beats past the row, past the
// pass or past the matrix read zeros through the buffer range checks.
template <int RT, int NT, int ST>
__device__ __forceinline__ void mfma_wave_tiles(const SmallBatchArgs &A, uint32_t rt0, uint32_t tok_group,
                                                uint32_t *lut, uint8_t *xl2, bool active) {
    const int lane = threadIdx.x & 63;
    const uint32_t lb = lut_lane_bits(lane);
    uint32_t lo_lane[4];  // this lane's offset within each quarter's operand
#pragma unroll
    for (int q = 0; q < 4; ++q) lo_lane[q] = lane_off(lane, q);
    const uint32_t tok = tok_group * kMfmaTokens + (lane & 15);
    // The epilogue's inputs, loaded first: the output pointers, the weight scale, the shape and the
    // token's scale (the empty asm keeps the compiler from sinking their loads to the stores). Loaded at
    // the end, their latencies stood before every tile's stores: 1.5-1.9 us on the decode-step set.
    // (With them the compiler waits for the step's own beats at the top of the streaming loop, before it
    // issues the next step's: no load of a later step is ever waited for in the loop.)
    int32_t *out_i32 = A.out_i32;
    float *out_f32 = A.out_f32;
    float w_scale = A.w_scale;
    int32_t rows = A.rows, batch = A.batch;
    asm volatile("" : "+s"(out_i32), "+s"(out_f32), "+s"(w_scale), "+s"(rows), "+s"(batch));
    const float xs_tok = A.x_scales[(int)tok < batch ? tok : 0u];
    const int g = lane >> 4, m = lane & 15;
    const bool lo = m < 8;
    const int bpr = A.bpr;
    const int n_steps = (bpr + 7) / 8;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(A.planes, A.plane_bytes);
    uint32_t row[RT][2];
    bool live[RT][2];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            row[t][j] = (rt0 + t) * kMfmaRows + 8 * j + (m & 7);
            live[t][j] = active && (int)row[t][j] < A.rows;
        }
    const int bj0 = g + (lo ? 0 : 4), bj1 = g + (lo ? 4 : 0);  // block of load 0 / 1 within a step
    v4i acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = v4i{0, 0, 0, 0};
    u32x4 bb[ST][RT][2];
    int s_end = 0;  // the current pass's end
    auto issue = [&](u32x4 (&beat)[RT][2], int st) {
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int b = 8 * st + (j ? bj1 : bj0);
                const bool in = st < s_end && b < bpr && live[t][j];
                beat[t][j] = load_beat(wr, in ? (row[t][j] * (uint32_t)bpr + (uint32_t)b) * 16u : kOutOfRange);
            }
    };
    // A step in two halves (its first iteration for every row tile, then its second), each with its
    // own four operands: 16 fewer registers live than reading all eight at once.
    auto step = [&](const u32x4 (&beat)[RT][2], int ls) {  // ls: the step's index within the pass
        const uint8_t *xs = op_base(lut, xl2, ls);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 xo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                xo[q] = *reinterpret_cast<const u32x4 *>(xs + lo_lane[q] + (4 * h + q) * kXtPieceStride);
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                const u32x4 p = h == 0 ? step_first(beat[t][0], beat[t][1], lo) : step_second(beat[t][0], beat[t][1], lo);
                acc[t] = mfma_beat_own(lut, p, xo, acc[t], lb);
            }
        }
    };
    for (int s0 = 0; s0 < n_steps || s0 == 0; s0 += kXtPassSteps) {
        s_end = min(n_steps, s0 + kXtPassSteps);
#pragma unroll
        for (int k = 0; k + 1 < ST; ++k) issue(bb[k], s0 + k);
        __syncthreads();  // the previous pass's operands are no longer read
        stage_x<NT>(lut, xl2, A, (int)(tok_group * kMfmaTokens), s0);
        __syncthreads();  // operands (and on the first pass the table) complete
        for (int st = s0; st < s_end; st += ST) {
#pragma unroll
            for (int k = 0; k < ST; ++k) {
                if (st + k >= s_end) break;  // wave-uniform: the pass has no step st + k
                issue(bb[(k + ST - 1) % ST], st + k + ST - 1);
                asm volatile("" ::: "memory");
                step(bb[k], st + k - s0);
            }
        }
        if (n_steps == 0) break;
    }
    // lane l, register i of row tile t: row 16 (rt0 + t) + 4 (l / 16) + i, token l % 16
    const int otok = (int)tok;
    if (!active || otok >= batch) return;
    const float xs = xs_tok;
    // Four consecutive rows of one token per lane: one 16-byte store per row tile and output where the
    // rows and both outputs allow it. Stored one word at a time, the outputs cost 21 us of the decode
    // step at 4 tokens and 45 us at 16 (measured with the stores removed): each instruction then
    // scattered 64 single words; with 16-byte stores the step took 8 and 23 us less.
    const bool vec = (rows & 3) == 0 &&
                     (((uintptr_t)out_i32 | (out_f32 ? (uintptr_t)out_f32 : (uintptr_t)0)) & 15u) == 0;
    if (vec) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int orow = (int)(rt0 + t) * kMfmaRows + 4 * (lane >> 4);
            if (orow < rows) {  // rows is a multiple of 4: the lane's four rows are all in, or all out
                const int64_t idx = (int64_t)otok * rows + orow;
                *reinterpret_cast<v4i *>(out_i32 + idx) = acc[t];
                if (out_f32) {
                    f32x4 f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) f[i] = ((float)acc[t][i] * xs) * w_scale;  // the scales in turn
                    *reinterpret_cast<f32x4 *>(out_f32 + idx) = f;
                }
            }
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int orow = (int)(rt0 + t) * kMfmaRows + 4 * (lane >> 4) + i;
            if (orow < rows) {
                const int64_t idx = (int64_t)otok * rows + orow;
                const int32_t sum = acc[t][i];
                out_i32[idx] = sum;
                if (out_f32) out_f32[idx] = ((float)sum * xs) * w_scale;  // the scales in turn
            }
        }
    }
}

__global__ __launch_bounds__(64 * kSBGroupWaves) void gemm_small_batch_mfma_grouped_kernel(
    const SmallBatchArgs *__restrict__ jobs, const SBTile *__restrict__ tiles) {
    __shared__ __attribute__((aligned(16))) uint32_t lut[kLutBytes / 4];
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const SBTile t = tiles[blockIdx.x];
    if (t.row_tile < 0) return;  // padding of the XCD runs (uniform over the workgroup)
    fill_lut_copies(lut, 64 * kSBGroupWaves);  // made visible by the first staging barrier
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const SmallBatchArgs &A = jobs[t.job];
    const uint32_t rt0 = (uint32_t)(t.row_tile * kSBGroupWaves * kSBWaveTiles + wave * kSBWaveTiles);
    const bool active = (int64_t)rt0 * kMfmaRows < A.rows;  // wave-uniform; idle waves still stage
    mfma_wave_tiles<kSBWaveTiles, 64 * kSBGroupWaves, kSBStages>(A, rt0, (uint32_t)t.tok_group, lut, smem,
                                                                 active);
}

// ------------------------------------------------------------------------------------------
// Launcher.

int launch_gemm_small_batch_mfma(const SmallBatchArgs &a, void *stream) {
    const unsigned row_wgs = (unsigned)((a.rows + kMfmaRows - 1) / kMfmaRows);
    const unsigned groups = (unsigned)((a.batch + kMfmaTokens - 1) / kMfmaTokens);
    if (row_wgs == 0 || groups == 0) return hipSuccess;
    if (a.bpr > 64)
        hipLaunchKernelGGL(gemm_small_batch_mfma_kernel<8>, dim3(row_wgs, groups), dim3(512), 0, as_stream(stream), a);
    else
        hipLaunchKernelGGL(gemm_small_batch_mfma_kernel<4>, dim3(row_wgs, groups), dim3(256), 0, as_stream(stream), a);
    return hipGetLastError();
}

int launch_gemm_small_batch_grouped(const SmallBatchArgs *jobs, const SBTile *tiles, int32_t n_tiles, void *stream) {
    if (n_tiles <= 0) return hipSuccess;
    const size_t lds = kSbGroupedLds;
    const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void *>(gemm_small_batch_mfma_grouped_kernel),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (ea != hipSuccess) return ea;
    hipLaunchKernelGGL(gemm_small_batch_mfma_grouped_kernel, dim3((unsigned)n_tiles), dim3(64 * kSBGroupWaves), lds,
                       as_stream(stream), jobs, tiles);
    return hipGetLastError();
}

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

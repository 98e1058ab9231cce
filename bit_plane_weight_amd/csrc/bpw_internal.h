// bpw_internal.h - device-side tables shared by the host dispatcher (bpw_host.cpp) and the
// kernels (bpw_*.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

struct bpw_host_mat;  // include/bpw.h

namespace bpw {

// Launch geometry of the ternary GEMV kernels.
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;     // wave64
constexpr int kKMaxBitSerial = 2;         // beats one lane holds per row-group (bit-serial kernels,
                                          // shapes other than 2560 and 6912 columns)
constexpr int kSBWaves = 16;              // waves of a small-batch workgroup (one row-group each)
constexpr int kSBThreads = 64 * kSBWaves;
constexpr int kXPassBlocks = 128;         // activation-plane blocks held in LDS per pass (8 KiB)
static_assert(kXPassBlocks == 64 * kKMaxBitSerial, "a wide row's pass is one full wave of lanes x kKMaxBitSerial");
constexpr int kTileRows = 1024;           // most rows of one bit-serial GEMV tile (its sums sit in LDS)
constexpr int kIters = 4;                 // row-iterations per wave per tile

// One GEMV of a grouped launch, as the kernels read it (lives in the caller's workspace).
struct DevJob {
    const uint8_t *planes;  // rows * bpr beats of 16 bytes
    const int8_t *x;        // activation codes, >= bpr * 64 bytes readable, 16-byte aligned
    int32_t *out_i32;
    float *out_f32;         // may be null
    int32_t rows;
    int32_t bpr;
    float x_scale;
    float w_scale;
    const float *x_scale_ptr;  // if set, the activation scale is read from here (x_scale ignored)
    int32_t glog;           // log2 of lanes per row (G)
    int32_t kblk;           // beats per lane per pass (0 when cols == 0)
    int32_t nchunk;         // passes over the row: bpr <= G * kblk * nchunk
    int32_t tile_rows;      // kWaves * kIters * (64 / G) (host bookkeeping; the kernels do not read it)
    uint32_t plane_bytes;   // rows * bpr * 16 (the buffer range of the weight loads)
    int32_t pair;           // 1: an IntMlp gate/up pair (planes = gate, out_i32 = gate sums or null)
    // IntMlp pairs only:
    const uint8_t *planes_up;  // up projection, same shape as the gate
    int32_t *out_up_i32;       // up sums or null
    int64_t *t_out;            // relu(a_g)^2 * a_u
    double *k_out;             // (S_g * S_g) * S_u
    float w_scale_up;
    int32_t pad;
};

// A tile of the bit-serial GEMV: consecutive row-groups ("units" of 64 / G rows) [u0, u1) of one
// job, at most kTileRows rows, run by one workgroup. In the batch-1 GEMV's tables the tile also
// carries copies of the job fields its first loads need (the other tables leave them zero), so that
// the beats and the activation leave after one record load instead of two dependent ones.
struct Tile {
    int32_t job;
    int32_t u0;
    int32_t u1;
    int32_t bpr;
    uint32_t plane_bytes;
    int32_t pair;
    const uint8_t *planes;
    const uint8_t *planes_up;
    const int8_t *x;
};
static_assert(sizeof(Tile) == 48, "tile records are 48 bytes");

// Host side: the tile of row-groups [u0, u1) of job `job`, job fields zero.
inline Tile tile_of(int32_t job, int64_t u0, int64_t u1) {
    Tile t{};
    t.job = job;
    t.u0 = (int32_t)u0;
    t.u1 = (int32_t)u1;
    return t;
}


// Small-batch arguments (passed by value; <= kMaxBatch tokens).
constexpr int kMaxBatch = 64;
constexpr int kSBMaxTokens = 16;  // tokens whose planes one small-batch workgroup holds in LDS (128 KiB)
struct SmallBatchArgs {
    const uint8_t *planes;
    const int8_t *X;          // [batch][ldx] int8 codes, 16-byte aligned rows
    int32_t *out_i32;         // [batch][rows]
    float *out_f32;           // [batch][rows] or null
    int64_t ldx;
    uint32_t plane_bytes;     // rows * bpr * 16 (the buffer range of the weight loads)
    uint32_t x_bytes;         // batch * ldx (the buffer range of the activation loads)
    int32_t rows, bpr, batch, glog, kblk, nchunk;
    int32_t tg;               // tokens per workgroup (<= kSBMaxTokens)
    float w_scale;
    float x_scales[kMaxBatch];
};

// A tile of the grouped small-batch launch: rows kSBGroupRows * row_tile .. +kSBGroupRows-1 and tokens
// 16 * tok_group .. +15 of call `job` (kSBGroupWaves waves x kSBWaveTiles row tiles of 16 rows).
// Measured on the decode-step set (B = 2 / 4 / 8 / 16, us): 8 waves x 2 tiles with two beat register
// sets and two workgroups per compute unit 146 / 150 / 158 / 174; 16 waves x 2 tiles, one workgroup per
// compute unit 149 / 152 / 158 / 178; 8 waves x 4 tiles with three or four sets 173-210; 8 x 3 (2 sets)
// 151-180; 8 x 2 with three sets 159-178.
constexpr int kSBGroupWaves = 8;
constexpr int kSBWaveTiles = 2;
constexpr int kSBStages = 2;  // beat register sets per wave (steps in flight + 1)
constexpr int kSBGroupRows = kSBGroupWaves * kSBWaveTiles * 16;
struct SBTile {
    int32_t job;
    int32_t row_tile;  // rows kSBGroupRows * row_tile ..; -1: an empty tile (padding of the XCD runs)
    int32_t tok_group;
    int32_t units;     // 1 (rows kSBGroupRows * row_tile .. + kSBGroupRows - 1); 0 for padding
};

// One GEMV of 2 to 4 tokens in the grouped small-batch launch (bit-serial; 2560 or 6912 columns).
// The tile table is the batch-1 one (Tile); a tile holds at most kTokTileRows rows.
constexpr int kTokMax = 4;
constexpr int kTokTileRows = 256;
struct TokJob {
    const uint8_t *planes;
    const int8_t *X;      // [batch][ldx]
    int32_t *out_i32;     // [batch][rows]
    float *out_f32;       // [batch][rows] or null
    int64_t ldx;
    uint32_t plane_bytes;
    int32_t rows, bpr;
    float w_scale;
    float x_scales[kTokMax];
};

// BITCOS GEMV launch geometry: 8 waves per workgroup (two workgroups per CU share the LDS, each
// holding the 64 KiB deposit table), tiles of kBcTileUnits row-groups. A row of bpr blocks is held by
// 2^glog lanes with k contiguous blocks each (k * 2^glog >= bpr); a row-group is the 64 >> glog rows
// one wave covers at a time.
constexpr int kBcWaves = 8;
constexpr int kBcThreads = 64 * kBcWaves;
constexpr int kBcTileUnits = 32;
struct BcGeometry {
    int k, glog;
};
constexpr BcGeometry bitcos_geometry(int64_t bpr) {
    return bpr <= 16 ? BcGeometry{2, 3} : bpr <= 40 ? BcGeometry{5, 3} : bpr <= 64 ? BcGeometry{4, 4} : BcGeometry{4, 5};
}

// One BITCOS GEMV of a grouped launch (lives in the caller's workspace).
struct BitcosJob {
    const uint64_t *presence;   // rows * bpr words
    const uint32_t *row_start;  // rows + 1 words
    const uint32_t *signs;
    const int8_t *x;
    int32_t *out_i32;
    float *out_f32;             // may be null
    int32_t rows, bpr;
    float x_scale, w_scale;
    uint32_t presence_bytes, row_start_bytes, sign_bytes;  // the buffer ranges
    int32_t pad;
};

// One activation of the Folded quantiser (lives in the caller's workspace).
struct QuantJob {
    const float *h;
    const float *g;
    int8_t *q;
    float *scale;
    int64_t n;
    int64_t q_len;
    float eps;
    int32_t pad;
};

// Host side (bpw_host.cpp): record the reason of a failing call for bpw_last_error(); a keyed hash
// of a device descriptor's fields (its seal); the gfx950 check; the XCD count of the current device;
// a tile table permuted so that each XCD runs one contiguous run of it; a validated host matrix's
// planes and shape.
void record_error(const char *msg);
uint64_t seal_words(const uint64_t *w, int n);
int host_check_device();  // a bpw_status
int host_xcds();
void host_xcd_layout(Tile *tiles, int64_t n);
const uint8_t *host_mat_view(const ::bpw_host_mat *m, int64_t *rows, int64_t *cols, float *w_scale);

// The fixed device scratch of bpw_gemv_noalloc (bpw_static.hip): kStaticScratchBytes per device, its
// device address looked up once per device. Returns a hipError_t.
constexpr size_t kStaticScratchBytes = size_t(1) << 20;
constexpr int kStaticMaxDevices = 64;
int static_scratch(void **ptr, size_t *len);

// Kernel launchers (bpw_*.hip). Each returns the hipError_t of its launch as int.
int launch_gemv_bytelane(const DevJob *jobs, const Tile *tiles, int32_t n_tiles, void *stream);
// bit-serial: workgroup w runs tiles[w]
int launch_gemv_bitserial(const DevJob *jobs, const Tile *tiles, int32_t n_tiles, void *stream);
int launch_gemm_small_batch(const SmallBatchArgs &a, int32_t row_wgs, int32_t token_groups, void *stream);
int launch_gemm_small_batch_mfma(const SmallBatchArgs &a, void *stream);
int launch_gemm_small_batch_grouped(const SmallBatchArgs *jobs, const SBTile *tiles, int32_t n_tiles, void *stream);
int launch_gemv_tokens(const TokJob *jobs, const Tile *tiles, int32_t n_tiles, int32_t nt, void *stream);
int launch_gemv_bitcos(const BitcosJob *jobs, const Tile *tiles, int32_t n_tiles, void *stream);
int launch_dense_head(const uint16_t *w, int64_t rows, int64_t cols, const uint16_t *x, float *y, void *stream);
int launch_quantize(const QuantJob *jobs, int32_t n_jobs, void *stream);
constexpr int32_t kProbeShapes = 5;
int launch_probe(const void *buf, size_t len, uint32_t *sink, int32_t shape, void *stream);
int launch_flush(void *buf, size_t len, void *stream);

}  // namespace bpw

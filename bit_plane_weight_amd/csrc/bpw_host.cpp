// bpw_host.cpp - host side of libbpw: argument checks, .trit v1 packing and validation,
// upload, grouped-GEMV planning and kernel dispatch. See include/bpw.h for the contract.
//
// Passages followed (cited by page title and section):
//   "The .trit format, version 1": 2.2 (scale finite and > 0), 2.3 (beat layout, P1, P2 with a
//   64-bit tail mask), section 4 (checks 15, 17, 18 and how violations are reported).
//   "Tritium: One Weight Format for Ternary Inference ...": "Invariants", "CPU kernels" (a pinned
//   kernel that cannot run is an error, never a fallback).
#include <hip/hip_runtime.h>
#include <emmintrin.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <random>
#include <string>
#include <vector>

#include "../../include/bpw.h"
#include "bpw_internal.h"

namespace {

thread_local std::string g_last_error;

bpw_status fail(bpw_status code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
bpw_status fail(bpw_status code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

}  // namespace

namespace bpw {
void record_error(const char *msg) { g_last_error = msg; }
}  // namespace bpw

namespace {

void set_err(bpw_err *e, bpw_status code, int64_t row, int64_t beat, int64_t col) {
    if (e) {
        e->code = code;
        e->row = row;
        e->beat = beat;
        e->col = col;
    }
}

inline int64_t beats_per_row(int64_t cols) { return (cols + 63) / 64; }

inline uint64_t load_le64(const uint8_t *p) {
    uint64_t v;
    std::memcpy(&v, p, 8);  // hosts that run ROCm are little-endian, as the format is
    return v;
}

inline void store_le64(uint8_t *p, uint64_t v) { std::memcpy(p, &v, 8); }

// Mask of valid columns in a row's last beat, built in 64 bits (format page 2.3, P2).
inline uint64_t tail_mask(int64_t cols) {
    const int r = (int)(cols % 64);
    return r == 0 ? ~UINT64_C(0) : ((UINT64_C(1) << r) - UINT64_C(1));
}

bool shape_ok(int64_t rows, int64_t cols) {
    // The kernels index one matrix's rows as int32, and rows * bpr * 16 (the plane bytes, compared with
    // the caller's length) must not wrap: a wrapped count could match a short buffer.
    if (rows < 0 || cols < 0 || rows > (int64_t)INT32_MAX || cols > ((int64_t)1 << 40)) return false;
    const int64_t bpr = (cols + 63) / 64;
    return bpr == 0 || rows <= (INT64_MAX / 16) / bpr;
}

// ---------------------------------------------------------------- descriptor seal

uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t seal_key() {
    static const uint64_t key = [] {
        std::random_device rd;
        uint64_t k = ((uint64_t)rd() << 32) ^ rd();
        k ^= (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        return mix64(k | 1);
    }();
    return key;
}

uint64_t seal_of(const bpw_dev_mat &m) {
    uint32_t sb;
    std::memcpy(&sb, &m.w_scale, 4);
    uint64_t h = seal_key();
    h = mix64(h ^ (uint64_t)(uintptr_t)m.d_planes);
    h = mix64(h ^ (uint64_t)m.rows);
    h = mix64(h ^ (uint64_t)m.cols);
    h = mix64(h ^ (uint64_t)m.bpr);
    h = mix64(h ^ (uint64_t)sb ^ ((uint64_t)m.reserved << 32));
    return h;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }

// ---------------------------------------------------------------- device check

std::atomic<int> g_arch_state[64];  // 0 unknown, 1 gfx950, 2 other

bpw_status check_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(BPW_E_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    const char *force = std::getenv("BPW_FORCE_ARCH_MISMATCH");  // test hook: can only make calls fail
    if (force && force[0] == '1') return fail(BPW_E_ARCH, "device %d: architecture check forced to fail", dev);
    const int slot = dev >= 0 && dev < 64 ? dev : -1;
    if (slot >= 0) {
        const int st = g_arch_state[slot].load(std::memory_order_acquire);
        if (st == 1) return BPW_OK;
        if (st == 2) return fail(BPW_E_ARCH, "device %d is not gfx950", dev);
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(BPW_E_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                    (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    if (slot >= 0) g_arch_state[slot].store(ok ? 1 : 2, std::memory_order_release);
    if (!ok) return fail(BPW_E_ARCH, "device %d is %s, not gfx950", dev, prop.gcnArchName);
    return BPW_OK;
}

// XCDs of the current device (hipDeviceAttributeNumberOfXccs; 1 if the runtime cannot say), cached
// per device. Workgroup b of a launch runs on XCD b mod this count.
std::atomic<int> g_xcds[64];
int device_xcds() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    const int slot = dev >= 0 && dev < 64 ? dev : -1;
    if (slot >= 0) {
        const int v = g_xcds[slot].load(std::memory_order_acquire);
        if (v > 0) return v;
    }
    int n = 1;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n < 1) n = 1;
    if (slot >= 0) g_xcds[slot].store(n, std::memory_order_release);
    return n;
}

// Compute units of the current device (1 if the runtime cannot say), cached per device.
std::atomic<int> g_cus[64];
int device_cus() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    const int slot = dev >= 0 && dev < 64 ? dev : -1;
    if (slot >= 0) {
        const int v = g_cus[slot].load(std::memory_order_acquire);
        if (v > 0) return v;
    }
    int n = 1;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 1;
    if (slot >= 0) g_cus[slot].store(n, std::memory_order_release);
    return n;
}

bpw_status hip_status(int e, const char *what) {
    if (e == hipSuccess) return BPW_OK;
    return fail(BPW_E_HIP, "%s: %s", what, hipGetErrorString((hipError_t)e));
}

// ---------------------------------------------------------------- packing / validation

// Pack one row. Returns the first bad column (or -1).
int64_t pack_row(const int8_t *w, int64_t cols, int64_t bpr, uint8_t *out) {
    const __m128i one = _mm_set1_epi8(1), mone = _mm_set1_epi8(-1), zero = _mm_setzero_si128();
    for (int64_t b = 0; b < bpr; ++b) {
        const int8_t *src = w + b * 64;
        uint64_t pos = 0, neg = 0;
        if ((b + 1) * 64 <= cols) {
            for (int q = 0; q < 4; ++q) {
                const __m128i v = _mm_loadu_si128(reinterpret_cast<const __m128i *>(src + 16 * q));
                const uint32_t p = (uint32_t)_mm_movemask_epi8(_mm_cmpeq_epi8(v, one));
                const uint32_t n = (uint32_t)_mm_movemask_epi8(_mm_cmpeq_epi8(v, mone));
                const uint32_t z = (uint32_t)_mm_movemask_epi8(_mm_cmpeq_epi8(v, zero));
                if ((p | n | z) != 0xFFFFu) {
                    for (int k = 0; k < 16; ++k) {
                        const int8_t x = src[16 * q + k];
                        if (x != 0 && x != 1 && x != -1) return b * 64 + 16 * q + k;
                    }
                }
                pos |= (uint64_t)p << (16 * q);
                neg |= (uint64_t)n << (16 * q);
            }
        } else {
            for (int64_t k = 0; b * 64 + k < cols; ++k) {
                const int8_t x = src[k];
                if (x == 1)
                    pos |= UINT64_C(1) << k;
                else if (x == -1)
                    neg |= UINT64_C(1) << k;
                else if (x != 0)
                    return b * 64 + k;
            }
        }
        store_le64(out + b * 16, pos);
        store_le64(out + b * 16 + 8, neg);
    }
    return -1;
}

bpw_status validate_planes(const uint8_t *planes, size_t len, int64_t rows, int64_t cols, bpw_err *err) {
    set_err(err, BPW_OK, -1, -1, -1);
    if (!shape_ok(rows, cols)) {
        set_err(err, BPW_E_INVAL, -1, -1, -1);
        return fail(BPW_E_INVAL, "bad shape rows=%lld cols=%lld", (long long)rows, (long long)cols);
    }
    const int64_t bpr = beats_per_row(cols);
    const uint64_t need = (uint64_t)rows * (uint64_t)bpr * 16u;
    if ((uint64_t)len != need) {
        set_err(err, BPW_E_SIZE, -1, -1, -1);
        return fail(BPW_E_SIZE, "plane bytes %zu != rows * bpr * 16 = %llu", len, (unsigned long long)need);
    }
    if (need && !planes) {
        set_err(err, BPW_E_INVAL, -1, -1, -1);
        return fail(BPW_E_INVAL, "planes is NULL");
    }
    const uint64_t tail = tail_mask(cols);
    for (int64_t r = 0; r < rows; ++r) {
        const uint8_t *row = planes + (size_t)r * (size_t)bpr * 16;
        uint64_t both = 0;
        for (int64_t b = 0; b < bpr; ++b) both |= load_le64(row + b * 16) & load_le64(row + b * 16 + 8);
        const uint64_t last_pos = bpr ? load_le64(row + (bpr - 1) * 16) : 0;
        const uint64_t last_neg = bpr ? load_le64(row + (bpr - 1) * 16 + 8) : 0;
        const uint64_t pad = (last_pos | last_neg) & ~tail;
        if (!both && !pad) continue;
        // slow path: locate the first offending beat of this row (P1 before P2 within a beat)
        for (int64_t b = 0; b < bpr; ++b) {
            const uint64_t p = load_le64(row + b * 16), n = load_le64(row + b * 16 + 8);
            if (p & n) {
                const int64_t col = 64 * b + __builtin_ctzll(p & n);
                set_err(err, BPW_E_P1_BOTH_BITS, r, b, col);
                return fail(BPW_E_P1_BOTH_BITS, "both planes set at row %lld beat %lld column %lld", (long long)r,
                            (long long)b, (long long)col);
            }
            if (b == bpr - 1 && ((p | n) & ~tail)) {
                const int64_t col = 64 * b + __builtin_ctzll((p | n) & ~tail);
                set_err(err, BPW_E_P2_PADDING, r, b, col);
                return fail(BPW_E_P2_PADDING, "padding bit set in row %lld (column %lld >= cols %lld)", (long long)r,
                            (long long)col, (long long)cols);
            }
        }
    }
    return BPW_OK;
}

}  // namespace

struct bpw_host_mat {
    uint8_t *planes;
    size_t bytes;
    int64_t rows, cols, bpr;
    float w_scale;
};

// ---------------------------------------------------------------- grouped GEMV plan

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct Geometry {
    int32_t glog, kblk, nchunk, tile_rows;
};

// Lanes per row G = 2^glog and beats per lane K, for the batch-1 kernels (bit-serial and byte-lane
// selects share the tiles) and the small batch: the two row widths of the model have compiled-in
// geometry (2560 columns: 8 lanes x 5 beats; 6912 columns: 32 lanes x 4 beats). Other widths take the
// smallest power-of-two G with ceil(bpr / G) <= kKMaxBitSerial for rows of up to kXPassBlocks blocks
// (one LDS pass); wider rows take passes of kXPassBlocks = 64 lanes x kKMaxBitSerial beats.
Geometry geometry_for(int64_t bpr) {
    Geometry g{0, 0, 0, 0};
    if (bpr == 0) {
        g.tile_rows = bpw::kWaves * bpw::kIters * 64;
        return g;
    }
    if (bpr == 40 || bpr == 108) {
        g.glog = bpr == 40 ? 3 : 5;
        g.kblk = bpr == 40 ? 5 : 4;
        g.nchunk = 1;
        g.tile_rows = bpw::kWaves * bpw::kIters * (int32_t)(64 >> g.glog);
        return g;
    }
    const int kmax = bpw::kKMaxBitSerial;
    int glog = 0;
    while (glog < 6 && ((bpr + (1 << glog) - 1) >> glog) > kmax) ++glog;
    int64_t G = (int64_t)1 << glog;
    int64_t k = (bpr + G - 1) / G;
    int64_t nchunk = 1;
    if (bpr > bpw::kXPassBlocks) {
        glog = 6;
        G = 64;
        k = bpw::kXPassBlocks / G;
        nchunk = (bpr + bpw::kXPassBlocks - 1) / bpw::kXPassBlocks;
    }
    g.glog = glog;
    g.kblk = (int32_t)k;
    g.nchunk = (int32_t)nchunk;
    g.tile_rows = bpw::kWaves * bpw::kIters * (int32_t)(64 >> glog);
    return g;
}

struct Layout {
    size_t jobs_off, work_off, total;
    int64_t n_work;  // tiles of the selected kernel
};

// Row-groups of one job for the bit-serial kernels: 64/G rows each (64 rows when cols == 0).
inline int64_t units_of(int64_t rows, const Geometry &g) {
    const int64_t rpi = 64 >> g.glog;
    return (rows + rpi - 1) / rpi;
}

// Row-groups in one bit-serial tile of a job: kTileUnits, or fewer where kTileRows caps the rows; a
// pair's tile holds half as many of each matrix. The plan then cuts the last kTailShare of each XCD's
// run of tiles into tiles of 1/kTailDiv the width (8 row-groups, two per wave), see xcd_runs.
constexpr int64_t kTileUnits = 32;
constexpr double kTailShare = 0.75;
constexpr int64_t kTailDiv = 4;
constexpr int64_t kMaxXcds = 64;  // bound on the XCD count used to size the workspace
inline int64_t tile_units(const Geometry &g) {
    return std::min<int64_t>(kTileUnits, bpw::kTileRows / (64 >> g.glog));
}

int64_t bitserial_tiles(const bpw_gemv_job &j) {
    const Geometry g = geometry_for(j.m.bpr);
    const int64_t tu = tile_units(g);
    return (units_of(j.m.rows, g) + tu - 1) / tu;
}

// An IntMlp pair's tiles: kPairTileUnits row-groups of each matrix (so as many beats as a plain
// tile of kTileUnits row-groups).
int64_t pair_tiles(const bpw_intmlp_job &j) {
    const Geometry g = geometry_for(j.gate.bpr);
    const int64_t tu = tile_units(g) / 2;
    return (units_of(j.gate.rows, g) + tu - 1) / tu;
}

// n_work counts the tiles before the tail split; total bounds the table after it: the split and the
// padding of the XCD runs (xcd_runs) give at most (n_work + kMaxXcds) * kTailDiv bit-serial tiles.
Layout layout_for(const bpw_gemv_job *jobs, int32_t n, const bpw_intmlp_job *mlp = nullptr, int32_t n_mlp = 0) {
    Layout L{};
    L.jobs_off = 0;
    L.n_work = 0;
    for (int32_t i = 0; i < n; ++i) L.n_work += bitserial_tiles(jobs[i]);
    for (int32_t i = 0; i < n_mlp; ++i) L.n_work += pair_tiles(mlp[i]);
    L.work_off = align_up(L.jobs_off + sizeof(bpw::DevJob) * (size_t)(n + n_mlp));
    const int64_t tile_bound = L.n_work > 0 ? (L.n_work + kMaxXcds) * kTailDiv : 0;
    L.total = align_up(L.work_off + sizeof(bpw::Tile) * (size_t)tile_bound);
    return L;
}

bpw_status check_dev_mat(const bpw_dev_mat *m, const char *who) {
    if (!m) return fail(BPW_E_INVAL, "%s: matrix descriptor is NULL", who);
    if (m->seal != seal_of(*m))
        return fail(BPW_E_NOT_VALIDATED, "%s: matrix descriptor was not produced by bpw_upload (or was modified)",
                    who);
    return BPW_OK;
}

bpw_status check_job(const bpw_gemv_job &j, int32_t i, const char *kind = "job") {
    char who[48];
    std::snprintf(who, sizeof who, "%s %d", kind, i);
    bpw_status st = check_dev_mat(&j.m, who);
    if (st) return st;
    const uint64_t bytes = (uint64_t)j.m.rows * (uint64_t)j.m.bpr * 16u;
    const Geometry g = geometry_for(j.m.bpr);
    if ((uint64_t)(j.m.rows + g.tile_rows) * (uint64_t)j.m.bpr * 16u >= 0xFFFFFFF0ull)
        return fail(BPW_E_UNSUPPORTED, "%s: %llu plane bytes exceed the 32-bit offsets of one matrix", who,
                    (unsigned long long)bytes);
    if (!j.d_x) return fail(BPW_E_INVAL, "%s: d_x is NULL", who);
    if (((uintptr_t)j.d_x & 15u) != 0) return fail(BPW_E_INVAL, "%s: d_x must be 16-byte aligned", who);
    if (j.x_len < j.m.bpr * 64)
        return fail(BPW_E_INVAL, "%s: x_len %lld < bpr * 64 = %lld", who, (long long)j.x_len,
                    (long long)(j.m.bpr * 64));
    if (!j.d_out_i32) return fail(BPW_E_INVAL, "%s: d_out_i32 is NULL", who);
    if (!std::isfinite(j.x_scale)) return fail(BPW_E_INVAL, "%s: x_scale is not finite", who);
    return BPW_OK;
}

// The dispatcher hands workgroup b of a launch to XCD b mod X in turn, and each XCD has its own L2
// and address-translation caches. Permuting the tile table so that XCD x runs one contiguous run of
// it (instead of every X-th tile) keeps the tiles an XCD streams at the same time on nearby
// addresses, and its activation vectors in its own L2. Measured on the decode-step set: 83.6 us with
// every X-th tile per XCD, 82.0 us with contiguous runs (a seeded shuffle of the tiles: 87.2 us).
template <class T>
void xcd_contiguous(T *tiles, int64_t n, int X) {
    if (X <= 1 || n <= X) return;
    std::vector<T> src(tiles, tiles + n);
    std::vector<int64_t> start(X + 1, 0);
    for (int x = 0; x < X; ++x) start[x + 1] = start[x] + (n - x + X - 1) / X;  // blocks b with b % X == x
    for (int64_t b = 0; b < n; ++b) tiles[b] = src[start[b % X] + b / X];
}

// The bit-serial table per XCD: XCD x runs one contiguous run of the job-ordered tiles (as
// xcd_contiguous), and the last kTailShare of each run is cut into tiles of 1/kTailDiv the width, so
// the large tiles go first and the run ends in small ones that finish close together. Runs are padded
// to one length with empty tiles (u0 == u1, no rows; they only stage the job's activation) and
// interleaved, workgroup b taking entry b / X of run b mod X. Returns the table length. Measured on
// the decode step, same box: tiles of 16 row-groups in job-ordered XCD runs 81.4-81.7 us; all 8
// 79.6; 16 with the last 62 % at 8 78.1-78.4; 32 with the last 75 % at 8 77.9; tails of 4, 6, 10 or
// 12 row-groups 80-91 (an odd share per wave, or too little work per tile).
int64_t xcd_runs(bpw::Tile *tiles, int64_t n, int X, double tail_share) {
    X = std::max(1, X);
    std::vector<bpw::Tile> src(tiles, tiles + n);
    std::vector<std::vector<bpw::Tile>> runs((size_t)X);
    size_t longest = 0;
    int64_t s0 = 0;
    for (int x = 0; x < X; ++x) {
        const int64_t len = (n - x + X - 1) / X;
        const int64_t fine_from = s0 + len - (int64_t)((double)len * tail_share + 0.5);
        for (int64_t i = s0; i < s0 + len; ++i) {
            const bpw::Tile b = src[(size_t)i];
            if (i < fine_from) {
                runs[(size_t)x].push_back(b);
                continue;
            }
            const int64_t w = std::max<int64_t>(1, (b.u1 - b.u0 + kTailDiv - 1) / kTailDiv);
            for (int64_t u = b.u0; u < b.u1; u += w)
                runs[(size_t)x].push_back(bpw::tile_of(b.job, u, std::min<int64_t>(b.u1, u + w)));
        }
        s0 += len;
        longest = std::max(longest, runs[(size_t)x].size());
    }
    const bpw::Tile pad = bpw::tile_of(n > 0 ? src[0].job : 0, 1, 1);
    int64_t t = 0;
    for (size_t k = 0; k < longest; ++k)
        for (int x = 0; x < X; ++x) tiles[t++] = k < runs[(size_t)x].size() ? runs[(size_t)x][k] : pad;
    return t;
}

// Widest pair whose t = relu(a_g)^2 * a_u cannot overflow int64: |a| <= 128 * cols < 2^21.
constexpr int64_t kPairMaxCols = 16383;

bpw_status check_pair(const bpw_intmlp_job &j, int32_t i) {
    char who[48];
    std::snprintf(who, sizeof who, "pair %d gate", i);
    bpw_status st = check_dev_mat(&j.gate, who);
    if (st) return st;
    std::snprintf(who, sizeof who, "pair %d up", i);
    st = check_dev_mat(&j.up, who);
    if (st) return st;
    std::snprintf(who, sizeof who, "pair %d", i);
    if (j.gate.rows != j.up.rows || j.gate.cols != j.up.cols)
        return fail(BPW_E_INVAL, "%s: gate is %lld x %lld, up is %lld x %lld", who, (long long)j.gate.rows,
                    (long long)j.gate.cols, (long long)j.up.rows, (long long)j.up.cols);
    if (j.gate.cols > kPairMaxCols)
        return fail(BPW_E_UNSUPPORTED, "%s: %lld columns; t is exact in int64 only up to %lld", who,
                    (long long)j.gate.cols, (long long)kPairMaxCols);
    // the same limits as a plain job over the gate (the up matrix has the same size)
    bpw_gemv_job g{};
    g.m = j.gate;
    g.d_x = j.d_x;
    g.x_len = j.x_len;
    g.x_scale = j.x_scale;
    g.d_out_i32 = reinterpret_cast<int32_t *>(j.d_t);  // only checked for NULL here
    st = check_job(g, i, "pair");
    if (st) return st;
    if (!j.d_t || ((uintptr_t)j.d_t & 7u)) return fail(BPW_E_INVAL, "%s: d_t is NULL or not 8-byte aligned", who);
    if (!j.d_k || ((uintptr_t)j.d_k & 7u)) return fail(BPW_E_INVAL, "%s: d_k is NULL or not 8-byte aligned", who);
    return BPW_OK;
}

}  // namespace

struct bpw_gemv_plan {
    int device;
    int32_t kernel;
    const bpw::DevJob *jobs;
    const bpw::Tile *tiles;        // one per workgroup (either select)
    int64_t n_tiles;
    int32_t has_work;
};

// ---------------------------------------------------------------- ABI

extern "C" {

int32_t bpw_abi_version(void) { return BPW_ABI_VERSION; }

const char *bpw_status_string(int32_t s) {
    switch (s) {
        case BPW_OK: return "BPW_OK";
        case BPW_E_INVAL: return "BPW_E_INVAL";
        case BPW_E_SIZE: return "BPW_E_SIZE";
        case BPW_E_P1_BOTH_BITS: return "BPW_E_P1_BOTH_BITS";
        case BPW_E_P2_PADDING: return "BPW_E_P2_PADDING";
        case BPW_E_NOT_VALIDATED: return "BPW_E_NOT_VALIDATED";
        case BPW_E_ARCH: return "BPW_E_ARCH";
        case BPW_E_HIP: return "BPW_E_HIP";
        case BPW_E_UNSUPPORTED: return "BPW_E_UNSUPPORTED";
        case BPW_E_FORMAT: return "BPW_E_FORMAT";
        default: return "unknown status";
    }
}

const char *bpw_last_error(void) { return g_last_error.c_str(); }

bpw_status bpw_device_check(void) { return check_device(); }

bpw_status bpw_pack_i8(const int8_t *w, int64_t rows, int64_t cols, uint8_t *planes, size_t planes_len,
                       bpw_err *err) {
    set_err(err, BPW_OK, -1, -1, -1);
    if (!shape_ok(rows, cols)) {
        set_err(err, BPW_E_INVAL, -1, -1, -1);
        return fail(BPW_E_INVAL, "bad shape rows=%lld cols=%lld", (long long)rows, (long long)cols);
    }
    const int64_t bpr = beats_per_row(cols);
    const uint64_t need = (uint64_t)rows * (uint64_t)bpr * 16u;
    if ((uint64_t)planes_len != need) {
        set_err(err, BPW_E_SIZE, -1, -1, -1);
        return fail(BPW_E_SIZE, "planes_len %zu != rows * bpr * 16 = %llu", planes_len, (unsigned long long)need);
    }
    if (need && (!w || !planes)) {
        set_err(err, BPW_E_INVAL, -1, -1, -1);
        return fail(BPW_E_INVAL, "NULL input or output");
    }
    // Tail beats read past `cols` only through the scalar path, so a row buffer of exactly cols
    // bytes is never overrun.
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t bad = pack_row(w + r * cols, cols, bpr, planes + (size_t)r * (size_t)bpr * 16);
        if (bad >= 0) {
            set_err(err, BPW_E_INVAL, r, bad / 64, bad);
            return fail(BPW_E_INVAL, "weight %d at row %lld column %lld is not in {-1, 0, +1}",
                        (int)w[r * cols + bad], (long long)r, (long long)bad);
        }
    }
    return BPW_OK;
}

bpw_status bpw_validate(const uint8_t *planes, size_t len, int64_t rows, int64_t cols, bpw_err *err) {
    return validate_planes(planes, len, rows, cols, err);
}

bpw_status bpw_load(const uint8_t *planes, size_t len, int64_t rows, int64_t cols, float w_scale,
                    bpw_host_mat **out, bpw_err *err) {
    set_err(err, BPW_OK, -1, -1, -1);
    if (!out) return fail(BPW_E_INVAL, "out is NULL");
    *out = nullptr;
    if (!scale_ok(w_scale)) {
        set_err(err, BPW_E_INVAL, -1, -1, -1);
        return fail(BPW_E_INVAL, "w_scale %g must be finite and > 0", (double)w_scale);
    }
    if (!shape_ok(rows, cols)) {
        set_err(err, BPW_E_INVAL, -1, -1, -1);
        return fail(BPW_E_INVAL, "bad shape rows=%lld cols=%lld", (long long)rows, (long long)cols);
    }
    const int64_t bpr = beats_per_row(cols);
    const uint64_t need = (uint64_t)rows * (uint64_t)bpr * 16u;
    if ((uint64_t)len != need) {
        set_err(err, BPW_E_SIZE, -1, -1, -1);
        return fail(BPW_E_SIZE, "plane bytes %zu != rows * bpr * 16 = %llu", len, (unsigned long long)need);
    }
    if (need && !planes) {
        set_err(err, BPW_E_INVAL, -1, -1, -1);
        return fail(BPW_E_INVAL, "planes is NULL");
    }
    auto *m = new (std::nothrow) bpw_host_mat;
    if (!m) return fail(BPW_E_INVAL, "out of host memory");
    m->bytes = (size_t)need;
    m->planes = need ? static_cast<uint8_t *>(std::aligned_alloc(64, align_up((size_t)need))) : nullptr;
    if (need && !m->planes) {
        delete m;
        return fail(BPW_E_INVAL, "out of host memory for %zu bytes", (size_t)need);
    }
    if (need) std::memcpy(m->planes, planes, (size_t)need);
    m->rows = rows;
    m->cols = cols;
    m->bpr = bpr;
    m->w_scale = w_scale;
    // validate the library's own copy, so later writes to the caller's buffer cannot matter
    bpw_status st = validate_planes(m->planes, m->bytes, rows, cols, err);
    if (st) {
        std::free(m->planes);
        delete m;
        return st;
    }
    *out = m;
    return BPW_OK;
}

void bpw_host_mat_free(bpw_host_mat *m) {
    if (!m) return;
    std::free(m->planes);
    delete m;
}

size_t bpw_host_mat_bytes(const bpw_host_mat *m) { return m ? m->bytes : 0; }

bpw_status bpw_upload(const bpw_host_mat *m, void *d_dst, size_t d_len, void *stream, bpw_dev_mat *out) {
    if (!m || !out) return fail(BPW_E_INVAL, "NULL matrix or output descriptor");
    std::memset(out, 0, sizeof *out);
    if (m->bytes && !d_dst) return fail(BPW_E_INVAL, "d_dst is NULL");
    if (d_len < m->bytes) return fail(BPW_E_SIZE, "d_len %zu < plane bytes %zu", d_len, m->bytes);
    if (((uintptr_t)d_dst & (kAlign - 1)) != 0) return fail(BPW_E_INVAL, "d_dst must be 256-byte aligned");
    bpw_status st = check_device();
    if (st) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (m->bytes) {
        st = hip_status(hipMemcpyAsync(d_dst, m->planes, m->bytes, hipMemcpyHostToDevice, s), "hipMemcpyAsync");
        if (st) return st;
        st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize");
        if (st) return st;
    }
    out->d_planes = d_dst;
    out->rows = m->rows;
    out->cols = m->cols;
    out->bpr = m->bpr;
    out->w_scale = m->w_scale;
    out->reserved = 0;
    out->seal = seal_of(*out);
    return BPW_OK;
}

size_t bpw_gemv_workspace_bytes(const bpw_gemv_job *jobs, int32_t n_jobs) {
    if (!jobs || n_jobs <= 0) return 0;
    return layout_for(jobs, n_jobs).total;
}

static bpw_status create_plan(const bpw_gemv_job *jobs, int32_t n_jobs, const bpw_intmlp_job *mlp, int32_t n_mlp,
                              int32_t kernel, void *d_ws, size_t ws_len, void *stream, bpw_gemv_plan **out) {
    if (!out) return fail(BPW_E_INVAL, "out is NULL");
    *out = nullptr;
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return fail(BPW_E_INVAL, "bad job list");
    if (n_mlp < 0 || (n_mlp > 0 && !mlp)) return fail(BPW_E_INVAL, "bad pair list");
    if ((int64_t)n_jobs + n_mlp > INT32_MAX) return fail(BPW_E_INVAL, "too many jobs");
    if (kernel != BPW_KERNEL_AUTO && kernel != BPW_KERNEL_BITSERIAL && kernel != BPW_KERNEL_BYTELANE)
        return fail(BPW_E_UNSUPPORTED, "unknown kernel %d", (int)kernel);
    if (kernel == BPW_KERNEL_BYTELANE && n_mlp > 0)
        return fail(BPW_E_UNSUPPORTED, "IntMlp pairs run on the bit-serial kernel only (pinned: byte-lane)");
    for (int32_t i = 0; i < n_jobs; ++i) {
        bpw_status st = check_job(jobs[i], i);
        if (st) return st;
    }
    for (int32_t i = 0; i < n_mlp; ++i) {
        bpw_status st = check_pair(mlp[i], i);
        if (st) return st;
    }
    const int32_t n_all = n_jobs + n_mlp;
    Layout L = layout_for(jobs, n_jobs, mlp, n_mlp);
    if (L.n_work > (int64_t)INT32_MAX)
        return fail(BPW_E_UNSUPPORTED, "too many tiles for one launch");
    const size_t need = bpw_gemv_intmlp_workspace_bytes(jobs, n_jobs, mlp, n_mlp);
    if (n_all > 0 && need > ws_len) return fail(BPW_E_SIZE, "workspace %zu bytes < required %zu", ws_len, need);
    if (n_all > 0 && !d_ws) return fail(BPW_E_INVAL, "d_ws is NULL");
    if (((uintptr_t)d_ws & (kAlign - 1)) != 0) return fail(BPW_E_INVAL, "d_ws must be 256-byte aligned");
    bpw_status st = check_device();
    if (st) return st;
    int dev = 0;
    (void)hipGetDevice(&dev);

    auto *plan = new (std::nothrow) bpw_gemv_plan;
    if (!plan) return fail(BPW_E_INVAL, "out of host memory");
    uint8_t *ws = static_cast<uint8_t *>(d_ws);
    plan->device = dev;
    plan->kernel = kernel;
    plan->jobs = reinterpret_cast<const bpw::DevJob *>(ws + L.jobs_off);
    plan->tiles = reinterpret_cast<const bpw::Tile *>(ws + L.work_off);
    plan->n_tiles = L.n_work;
    plan->has_work = 0;
    if (n_all == 0) {
        *out = plan;
        return BPW_OK;
    }

    const size_t table_bytes = L.total;
    std::vector<uint8_t> host(table_bytes, 0);
    auto *hj = reinterpret_cast<bpw::DevJob *>(host.data() + L.jobs_off);
    auto *hb = reinterpret_cast<bpw::Tile *>(host.data() + L.work_off);
    // Tile-table order: the plain jobs in the order given, with the pairs merged in where their
    // share of the pairs' bytes matches the plain jobs' share so far (for a decode step: each layer's
    // pair beside its other projections). With the table laid out per XCD below, this gives every
    // XCD the same mix of shapes.
    std::vector<int32_t> order;
    order.reserve(n_all);
    {
        double tot_j = 0, tot_p = 0, done_j = 0, done_p = 0;
        for (int32_t i = 0; i < n_jobs; ++i) tot_j += (double)jobs[i].m.rows * (double)jobs[i].m.bpr;
        for (int32_t i = 0; i < n_mlp; ++i) tot_p += 2.0 * (double)mlp[i].gate.rows * (double)mlp[i].gate.bpr;
        int32_t a = 0, b = 0;
        while (a < n_jobs || b < n_mlp) {
            const bool take_pair = b < n_mlp && (a >= n_jobs || done_p * tot_j <= done_j * tot_p);
            if (take_pair) {
                done_p += 2.0 * (double)mlp[b].gate.rows * (double)mlp[b].gate.bpr;
                order.push_back(n_jobs + b++);
            } else {
                done_j += (double)jobs[a].m.rows * (double)jobs[a].m.bpr;
                order.push_back(a++);
            }
        }
    }
    int64_t t = 0;
    for (const int32_t i : order) {
        const bool pair = i >= n_jobs;
        const bpw_dev_mat &m = pair ? mlp[i - n_jobs].gate : jobs[i].m;
        const Geometry g = geometry_for(m.bpr);
        bpw::DevJob d{};
        d.planes = static_cast<const uint8_t *>(m.d_planes);
        d.rows = (int32_t)m.rows;
        d.bpr = (int32_t)m.bpr;
        d.w_scale = m.w_scale;
        d.glog = g.glog;
        d.kblk = g.kblk;
        d.nchunk = g.nchunk;
        d.tile_rows = g.tile_rows;
        d.plane_bytes = (uint32_t)((uint64_t)m.rows * (uint64_t)m.bpr * 16u);
        if (!pair) {
            const bpw_gemv_job &j = jobs[i];
            d.x = j.d_x;
            d.out_i32 = j.d_out_i32;
            d.out_f32 = j.d_out_f32;
            d.x_scale = j.x_scale;
            d.x_scale_ptr = j.d_x_scale;
        } else {
            const bpw_intmlp_job &j = mlp[i - n_jobs];
            d.pair = 1;
            d.x = j.d_x;
            d.out_i32 = j.d_gate_i32;
            d.x_scale = j.x_scale;
            d.x_scale_ptr = j.d_x_scale;
            d.planes_up = static_cast<const uint8_t *>(j.up.d_planes);
            d.out_up_i32 = j.d_up_i32;
            d.t_out = j.d_t;
            d.k_out = j.d_k;
            d.w_scale_up = j.up.w_scale;
        }
        hj[i] = d;
        // tiles of one job in row order, jobs in the order above (the whole table is then laid out per
        // XCD, below)
        const int64_t U = units_of(m.rows, g), tu = pair ? tile_units(g) / 2 : tile_units(g);
        for (int64_t u = 0; u < U; u += tu) hb[t++] = bpw::tile_of(i, u, std::min(U, u + tu));
        if (m.rows > 0) plan->has_work = 1;  // a job without rows has no tiles (a pair: not even K)
    }
    if (t != L.n_work) {
        delete plan;
        return fail(BPW_E_UNSUPPORTED, "internal: %lld tiles written, %lld expected", (long long)t, (long long)L.n_work);
    }
    const int xccs = device_xcds();
    if (xccs > kMaxXcds) {
        delete plan;
        return fail(BPW_E_UNSUPPORTED, "device has %d XCDs; the tile table is sized for %lld", xccs,
                    (long long)kMaxXcds);
    }
    // a plan too small to give every CU two wide tiles (one layer: 119) takes only narrow ones
    const double share = t < 2 * (int64_t)device_cus() ? 1.0 : kTailShare;
    plan->n_tiles = xcd_runs(hb, t, xccs, share);
    if (plan->n_tiles > (int64_t)INT32_MAX) {
        delete plan;
        return fail(BPW_E_UNSUPPORTED, "too many tiles for one launch");
    }
    for (int64_t k = 0; k < plan->n_tiles; ++k) {  // the job fields the tile's first loads need
        bpw::Tile &b = hb[k];
        const bpw::DevJob &d = hj[b.job];
        b.bpr = d.bpr;
        b.plane_bytes = d.plane_bytes;
        b.pair = d.pair;
        b.planes = d.planes;
        b.planes_up = d.planes_up;
        b.x = d.x;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    st = hip_status(hipMemcpyAsync(d_ws, host.data(), table_bytes, hipMemcpyHostToDevice, s), "hipMemcpyAsync");
    if (!st) st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize");
    if (st) {
        delete plan;
        return st;
    }
    *out = plan;
    return BPW_OK;
}

bpw_status bpw_gemv_plan_create(const bpw_gemv_job *jobs, int32_t n_jobs, int32_t kernel, void *d_ws,
                                size_t ws_len, void *stream, bpw_gemv_plan **out) {
    return create_plan(jobs, n_jobs, nullptr, 0, kernel, d_ws, ws_len, stream, out);
}

size_t bpw_gemv_intmlp_workspace_bytes(const bpw_gemv_job *jobs, int32_t n_jobs, const bpw_intmlp_job *mlp,
                                       int32_t n_mlp) {
    if (n_mlp <= 0 || !mlp) return bpw_gemv_workspace_bytes(jobs, n_jobs);
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return 0;
    return layout_for(jobs, n_jobs, mlp, n_mlp).total;
}

bpw_status bpw_gemv_intmlp_plan_create(const bpw_gemv_job *jobs, int32_t n_jobs, const bpw_intmlp_job *mlp,
                                       int32_t n_mlp, int32_t kernel, void *d_ws, size_t ws_len, void *stream,
                                       bpw_gemv_plan **out) {
    return create_plan(jobs, n_jobs, mlp, n_mlp, kernel, d_ws, ws_len, stream, out);
}

static bpw_status plan_ready(const bpw_gemv_plan *plan) {
    if (!plan) return fail(BPW_E_INVAL, "plan is NULL");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
        return fail(BPW_E_INVAL, "plan was created on device %d, current device is %d", plan->device, dev);
    return check_device();
}

bpw_status bpw_gemv_plan_run(const bpw_gemv_plan *plan, void *stream) {
    bpw_status st = plan_ready(plan);
    if (st) return st;
    if (!plan->has_work) return BPW_OK;
    if (plan->kernel == BPW_KERNEL_BYTELANE)
        return hip_status(bpw::launch_gemv_bytelane(plan->jobs, plan->tiles,
                                                    (int32_t)plan->n_tiles, stream),
                          "gemv launch");
    return hip_status(bpw::launch_gemv_bitserial(plan->jobs, plan->tiles,
                                                 (int32_t)plan->n_tiles, stream),
                      "gemv launch");
}

void bpw_gemv_plan_free(bpw_gemv_plan *plan) { delete plan; }

bpw_status bpw_gemv(const bpw_gemv_job *jobs, int32_t n_jobs, int32_t kernel, void *d_ws, size_t ws_len,
                    void *stream) {
    if (n_jobs == 0) return BPW_OK;
    bpw_gemv_plan *plan = nullptr;
    bpw_status st = bpw_gemv_plan_create(jobs, n_jobs, kernel, d_ws, ws_len, stream, &plan);
    if (st) return st;
    st = bpw_gemv_plan_run(plan, stream);
    bpw_gemv_plan_free(plan);
    return st;
}

bpw_status bpw_gemv_noalloc(const bpw_gemv_job *jobs, int32_t n_jobs, int32_t kernel, void *stream) {
    if (n_jobs == 0) return BPW_OK;
    if (n_jobs < 0 || !jobs) return fail(BPW_E_INVAL, "bad job list");
    bpw_status st = check_device();
    if (st) return st;
    void *ws = nullptr;
    size_t cap = 0;
    st = hip_status(bpw::static_scratch(&ws, &cap), "static scratch lookup (hipGetSymbolAddress)");
    if (st) return st;
    const size_t need = bpw_gemv_workspace_bytes(jobs, n_jobs);
    if (need > cap)
        return fail(BPW_E_SIZE, "bpw_gemv_noalloc: these jobs need %zu bytes of tables, the static scratch holds %zu",
                    need, cap);
    return bpw_gemv(jobs, n_jobs, kernel, ws, cap, stream);
}

struct bpw_quant_plan {
    int device;
    const bpw::QuantJob *jobs;
    int32_t n_jobs;
};

size_t bpw_quantize_workspace_bytes(int32_t n_jobs) {
    return n_jobs > 0 ? align_up(sizeof(bpw::QuantJob) * (size_t)n_jobs) : 0;
}

bpw_status bpw_quant_plan_create(const bpw_quant_job *jobs, int32_t n_jobs, void *d_ws, size_t ws_len, void *stream,
                                 bpw_quant_plan **out) {
    if (!out) return fail(BPW_E_INVAL, "out is NULL");
    *out = nullptr;
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return fail(BPW_E_INVAL, "bad quantiser job list");
    std::vector<bpw::QuantJob> table((size_t)n_jobs);
    for (int32_t i = 0; i < n_jobs; ++i) {
        const bpw_quant_job &j = jobs[i];
        if (!j.d_h || !j.d_g || !j.d_q || !j.d_scale)
            return fail(BPW_E_INVAL, "quantiser job %d: NULL pointer", (int)i);
        if (j.n < 1 || j.q_len < j.n) return fail(BPW_E_INVAL, "quantiser job %d: need 1 <= n <= q_len", (int)i);
        if (!std::isfinite(j.eps) || j.eps < 0.0f)
            return fail(BPW_E_INVAL, "quantiser job %d: eps must be finite and >= 0", (int)i);
        table[(size_t)i] = bpw::QuantJob{j.d_h, j.d_g, j.d_q, j.d_scale, j.n, j.q_len, j.eps, 0};
    }
    const size_t need = bpw_quantize_workspace_bytes(n_jobs);
    if (ws_len < need) return fail(BPW_E_SIZE, "workspace %zu bytes < required %zu", ws_len, need);
    if (need && (!d_ws || ((uintptr_t)d_ws & (kAlign - 1)) != 0))
        return fail(BPW_E_INVAL, "d_ws must be non-NULL and 256-byte aligned");
    bpw_status st = check_device();
    if (st) return st;
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (need) {
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        st = hip_status(hipMemcpyAsync(d_ws, table.data(), sizeof(bpw::QuantJob) * table.size(), hipMemcpyHostToDevice, s),
                        "hipMemcpyAsync");
        if (!st) st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize");
        if (st) return st;
    }
    auto *plan = new (std::nothrow) bpw_quant_plan;
    if (!plan) return fail(BPW_E_INVAL, "out of host memory");
    plan->device = dev;
    plan->jobs = static_cast<const bpw::QuantJob *>(d_ws);
    plan->n_jobs = n_jobs;
    *out = plan;
    return BPW_OK;
}

bpw_status bpw_quant_plan_run(const bpw_quant_plan *plan, void *stream) {
    if (!plan) return fail(BPW_E_INVAL, "plan is NULL");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
        return fail(BPW_E_INVAL, "plan was created on device %d, current device is %d", plan->device, dev);
    bpw_status st = check_device();
    if (st) return st;
    return hip_status(bpw::launch_quantize(plan->jobs, plan->n_jobs, stream), "quantiser launch");
}

void bpw_quant_plan_free(bpw_quant_plan *plan) { delete plan; }

bpw_status bpw_quantize(const bpw_quant_job *jobs, int32_t n_jobs, void *d_ws, size_t ws_len, void *stream) {
    if (n_jobs == 0) return BPW_OK;
    bpw_quant_plan *plan = nullptr;
    bpw_status st = bpw_quant_plan_create(jobs, n_jobs, d_ws, ws_len, stream, &plan);
    if (st) return st;
    st = bpw_quant_plan_run(plan, stream);
    bpw_quant_plan_free(plan);
    return st;
}

// BPW_KERNEL_AUTO takes the matrix-core kernel from this batch size on. Measured on MI355X at the
// gate/up and down shapes it is the faster one from batch 1 (4.8 us against 5.1-5.4 us) to 16
// (6.9-7.8 us against 12.3-17.9 us).
constexpr int32_t kMfmaFromBatch = 1;

// Argument checks of one small-batch call (shared by the single call and the grouped plan).
static bpw_status check_small_batch(const bpw_dev_mat *m, const int8_t *d_X, int32_t batch, int64_t ldx,
                                    const float *x_scales, const int32_t *d_out_i32, const char *who) {
    bpw_status st = check_dev_mat(m, who);
    if (st) return st;
    if (batch < 1 || batch > bpw::kMaxBatch) return fail(BPW_E_INVAL, "%s: batch %d outside [1, 64]", who, (int)batch);
    if (!d_X || !x_scales || !d_out_i32) return fail(BPW_E_INVAL, "%s: NULL argument", who);
    if (ldx < m->bpr * 64)
        return fail(BPW_E_INVAL, "%s: ldx %lld < bpr * 64 = %lld", who, (long long)ldx, (long long)(m->bpr * 64));
    if ((ldx % 16) != 0 || ((uintptr_t)d_X & 15u) != 0)
        return fail(BPW_E_INVAL, "%s: X rows must be 16-byte aligned (X aligned, ldx %% 16 == 0)", who);
    if ((uint64_t)(batch + 16) * (uint64_t)ldx >= 0xFFFFFFF0ull)
        return fail(BPW_E_UNSUPPORTED, "%s: (batch + 16) * ldx exceeds the 32-bit offsets of X", who);
    for (int32_t t = 0; t < batch; ++t)
        if (!std::isfinite(x_scales[t])) return fail(BPW_E_INVAL, "%s: x_scales[%d] is not finite", who, (int)t);
    if ((uint64_t)(m->rows + 64) * (uint64_t)m->bpr * 16u >= 0xFFFFFFF0ull)
        return fail(BPW_E_UNSUPPORTED, "%s: plane bytes exceed the 32-bit offsets of one matrix", who);
    return BPW_OK;
}

static bpw::SmallBatchArgs small_batch_args(const bpw_dev_mat *m, const int8_t *d_X, int32_t batch, int64_t ldx,
                                            const float *x_scales, int32_t *d_out_i32, float *d_out_f32) {
    const Geometry g = geometry_for(m->bpr);
    bpw::SmallBatchArgs a{};
    a.planes = static_cast<const uint8_t *>(m->d_planes);
    a.X = d_X;
    a.out_i32 = d_out_i32;
    a.out_f32 = d_out_f32;
    a.ldx = ldx;
    a.plane_bytes = (uint32_t)((uint64_t)m->rows * (uint64_t)m->bpr * 16u);
    a.x_bytes = (uint32_t)((uint64_t)batch * (uint64_t)ldx);
    a.rows = (int32_t)m->rows;
    a.bpr = (int32_t)m->bpr;
    a.batch = batch;
    a.glog = g.glog;
    a.kblk = g.kblk;
    a.nchunk = g.nchunk;
    a.w_scale = m->w_scale;
    for (int32_t t = 0; t < batch; ++t) a.x_scales[t] = x_scales[t];
    return a;
}

bpw_status bpw_gemm_small_batch(const bpw_dev_mat *m, const int8_t *d_X, int32_t batch, int64_t ldx,
                                const float *x_scales, int32_t *d_out_i32, float *d_out_f32, int32_t kernel,
                                void *stream) {
    if (kernel != BPW_KERNEL_AUTO && kernel != BPW_KERNEL_BITSERIAL && kernel != BPW_KERNEL_MFMA) {
        bpw_status st = check_dev_mat(m, "small batch");
        if (st) return st;
        return fail(BPW_E_UNSUPPORTED, "small batch: kernel %d is not available for this entry point", (int)kernel);
    }
    bpw_status st = check_small_batch(m, d_X, batch, ldx, x_scales, d_out_i32, "small batch");
    if (st) return st;
    const Geometry g = geometry_for(m->bpr);
    st = check_device();
    if (st) return st;
    if (m->rows == 0) return BPW_OK;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return fail(BPW_E_HIP, "small batch: could not read the compute-unit count");
    // Grid: kSBWaves row-groups per workgroup; tokens split into groups only as far as needed to give
    // every compute unit a workgroup (each group re-reads the weights, from the cache after the
    // first), and into groups of at most kSBMaxTokens (their planes sit in LDS).
    const int64_t rgs = units_of(m->rows, g);
    const int64_t row_wgs = (rgs + bpw::kSBWaves - 1) / bpw::kSBWaves;
    int64_t groups = std::max<int64_t>((batch + bpw::kSBMaxTokens - 1) / bpw::kSBMaxTokens, (cus + row_wgs - 1) / row_wgs);
    groups = std::min<int64_t>(groups, batch);
    const int64_t tg = (batch + groups - 1) / groups;
    groups = (batch + tg - 1) / tg;
    bpw::SmallBatchArgs a = small_batch_args(m, d_X, batch, ldx, x_scales, d_out_i32, d_out_f32);
    a.tg = (int32_t)tg;
    if (row_wgs > (int64_t)INT32_MAX) return fail(BPW_E_UNSUPPORTED, "small batch: too many rows for one launch");
    const bool mfma = kernel == BPW_KERNEL_MFMA || (kernel == BPW_KERNEL_AUTO && batch >= kMfmaFromBatch);
    if (mfma) return hip_status(bpw::launch_gemm_small_batch_mfma(a, stream), "small batch launch");
    return hip_status(bpw::launch_gemm_small_batch(a, (int32_t)row_wgs, (int32_t)groups, stream), "small batch launch");
}

// ---------------------------------------------------------------- grouped small batch

struct bpw_sb_plan {
    int device;
    const bpw::SmallBatchArgs *jobs;
    const bpw::SBTile *tiles;
    int64_t n_tiles;
    bpw_gemv_plan *gemv;  // batch 1 under AUTO: the batch-1 grouped GEMV over the same jobs
    // 2 to 4 tokens on the bit-serial kernel: its job and tile tables (n_tok_tiles > 0)
    const bpw::TokJob *tok_jobs;
    const bpw::Tile *tok_tiles;
    int64_t n_tok_tiles;
    int32_t nt;
};

namespace {
struct SBLayout {
    size_t jobs_off, tiles_off, total;
    int64_t n_tiles;
};

// Tiles of a grouped small-batch job per token group: kSBGroupRows rows each.
inline int64_t sb_job_tiles(const bpw_sb_job &j) { return (j.m.rows + bpw::kSBGroupRows - 1) / bpw::kSBGroupRows; }

// Table entries the grouped small-batch plan may write for n work tiles: the cost-balanced XCD runs
// below are padded to the longest run; beyond this bound the plan keeps equal-count runs.
inline int64_t sb_tile_bound(int64_t n) { return n > 0 ? 2 * n + kMaxXcds : 0; }

// Lay the job-ordered tiles of the grouped small batch out per XCD. The workgroups of one tile differ
// in cost (a 6912-column tile streams 2.7 times the beats of a 2560-column one) and every tile pays a
// fixed start (table, operand staging) and end; measured at 4 tokens on the decode-step set, a
// 256-row tile took about 6.8 us + 1.05 ns per row-beat (17.5 us at 2560 columns, 35.7 at 6912). The
// job-ordered table is cut into X contiguous runs of equal estimated cost (so each job's operands stay
// in one XCD's L2), each run is ordered longest tile first (the run then ends in short tiles), and
// runs are padded with empty tiles (row_tile -1: the workgroup exits at once) and interleaved,
// workgroup b taking entry b / X of run b mod X. With equal-count runs the XCDs finished 21 us apart.
// Returns the table length, or n (equal-count runs, xcd_contiguous) if the padded runs would not fit.
int64_t sb_cost_runs(bpw::SBTile *tiles, int64_t n, int X, const bpw_sb_job *jobs, int64_t cap) {
    X = std::max(1, X);
    auto cost = [&](const bpw::SBTile &t) {
        const bpw_sb_job &j = jobs[t.job];
        const int64_t r0 = (int64_t)t.row_tile * bpw::kSBGroupRows;
        const int64_t rows = std::min<int64_t>((int64_t)t.units * bpw::kSBGroupRows, j.m.rows - r0);
        return 6500.0 + (double)rows * (double)j.m.bpr;
    };
    double total = 0.0;
    for (int64_t i = 0; i < n; ++i) total += cost(tiles[i]);
    std::vector<std::vector<bpw::SBTile>> runs((size_t)X);
    double acc = 0.0;
    size_t longest = 0;
    for (int64_t i = 0, x = 0; i < n; ++i) {
        const double c = cost(tiles[i]);
        // start the next run once this one holds its share (the midpoint of the tile decides)
        while (x + 1 < X && acc + 0.5 * c > total * (double)(x + 1) / (double)X) ++x;
        runs[(size_t)x].push_back(tiles[i]);
        acc += c;
    }
    for (auto &r : runs) {
        std::stable_sort(r.begin(), r.end(),
                         [&](const bpw::SBTile &a, const bpw::SBTile &b) { return cost(a) > cost(b); });
        longest = std::max(longest, r.size());
    }
    if ((int64_t)(longest * (size_t)X) > cap) {
        xcd_contiguous(tiles, n, X);
        return n;
    }
    int64_t t = 0;
    for (size_t k = 0; k < longest; ++k)
        for (int x = 0; x < X; ++x)
            tiles[t++] = k < runs[(size_t)x].size() ? runs[(size_t)x][k] : bpw::SBTile{0, -1, 0, 0};  // padding
    return t;
}

// The grouped matrix-core launch's workspace: job records, then the tile table with room for the
// cost-balanced XCD runs padded to one length (sb_cost_runs).
SBLayout sb_layout(const bpw_sb_job *jobs, int32_t n, int32_t batch) {
    SBLayout L{};
    const int64_t groups = (batch + 15) / 16;
    for (int32_t i = 0; i < n; ++i) L.n_tiles += sb_job_tiles(jobs[i]) * groups;
    L.jobs_off = 0;
    L.tiles_off = align_up(sizeof(bpw::SmallBatchArgs) * (size_t)n);
    L.total = align_up(L.tiles_off + sizeof(bpw::SBTile) * (size_t)sb_tile_bound(L.n_tiles));
    return L;
}
}  // namespace

// The bit-serial token kernel serves 2 to 4 tokens of matrices 2560 or 6912 columns wide (40 or 108
// beats per row); its tables: one TokJob per job, tiles as the batch-1 plan cuts them (rows per tile
// capped at kTokTileRows), the same bound for the XCD runs.
namespace {
bool tok_shape(const bpw_dev_mat &m) { return m.bpr == 40 || m.bpr == 108; }

bool tok_ok(const bpw_sb_job *jobs, int32_t n, int32_t batch) {
    if (batch < 2 || batch > bpw::kTokMax) return false;
    for (int32_t i = 0; i < n; ++i)
        if (!tok_shape(jobs[i].m)) return false;
    return true;
}

inline int64_t tok_tile_units(const Geometry &g) {
    return std::min<int64_t>(kTileUnits, bpw::kTokTileRows / (64 >> g.glog));
}

int64_t tok_base_tiles(const bpw_sb_job *jobs, int32_t n) {
    int64_t t = 0;
    for (int32_t i = 0; i < n; ++i) {
        const Geometry g = geometry_for(jobs[i].m.bpr);
        const int64_t tu = tok_tile_units(g);
        t += (units_of(jobs[i].m.rows, g) + tu - 1) / tu;
    }
    return t;
}

SBLayout tok_layout(const bpw_sb_job *jobs, int32_t n) {
    SBLayout L{};
    L.n_tiles = tok_base_tiles(jobs, n);
    L.jobs_off = 0;
    L.tiles_off = align_up(sizeof(bpw::TokJob) * (size_t)n);
    const int64_t bound = L.n_tiles > 0 ? (L.n_tiles + kMaxXcds) * kTailDiv : 0;
    L.total = align_up(L.tiles_off + sizeof(bpw::Tile) * (size_t)bound);
    return L;
}
}  // namespace

// A small-batch job at batch 1 as a batch-1 GEMV job (the same sums and the same dequantisation).
static std::vector<bpw_gemv_job> sb_as_gemv(const bpw_sb_job *jobs, int32_t n) {
    std::vector<bpw_gemv_job> g((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        g[i] = bpw_gemv_job{};
        g[i].m = jobs[i].m;
        g[i].d_x = jobs[i].d_X;
        g[i].x_len = jobs[i].ldx;
        g[i].x_scale = jobs[i].x_scales ? jobs[i].x_scales[0] : 0.0f;
        g[i].d_out_i32 = jobs[i].d_out_i32;
        g[i].d_out_f32 = jobs[i].d_out_f32;
    }
    return g;
}

size_t bpw_gemm_small_batch_workspace_bytes(const bpw_sb_job *jobs, int32_t n_jobs, int32_t batch) {
    if (!jobs || n_jobs <= 0 || batch < 1) return 0;
    size_t need = sb_layout(jobs, n_jobs, batch).total;
    if (tok_ok(jobs, n_jobs, batch)) need = std::max(need, tok_layout(jobs, n_jobs).total);
    if (batch == 1) {
        const std::vector<bpw_gemv_job> g = sb_as_gemv(jobs, n_jobs);
        need = std::max(need, bpw_gemv_workspace_bytes(g.data(), n_jobs));
    }
    return need;
}

bpw_status bpw_gemm_small_batch_plan_create(const bpw_sb_job *jobs, int32_t n_jobs, int32_t batch, int32_t kernel,
                                            void *d_ws, size_t ws_len, void *stream, bpw_sb_plan **out) {
    if (!out) return fail(BPW_E_INVAL, "out is NULL");
    *out = nullptr;
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return fail(BPW_E_INVAL, "bad job list");
    if (kernel != BPW_KERNEL_AUTO && kernel != BPW_KERNEL_MFMA && kernel != BPW_KERNEL_BITSERIAL)
        return fail(BPW_E_UNSUPPORTED, "grouped small batch: unknown kernel %d", (int)kernel);
    if (batch < 1 || batch > bpw::kMaxBatch) return fail(BPW_E_INVAL, "batch %d outside [1, 64]", (int)batch);
    if (kernel == BPW_KERNEL_BITSERIAL && batch > 1 && !tok_ok(jobs, n_jobs, batch))
        return fail(BPW_E_UNSUPPORTED,
                    "grouped small batch, bit-serial: 2 to %d tokens of 2560- or 6912-column matrices only (pinned: "
                    "bit-serial)", bpw::kTokMax);
    char who[48];
    for (int32_t i = 0; i < n_jobs; ++i) {
        std::snprintf(who, sizeof who, "small-batch job %d", i);
        const bpw_sb_job &j = jobs[i];
        bpw_status st = check_small_batch(&j.m, j.d_X, batch, j.ldx, j.x_scales, j.d_out_i32, who);
        if (st) return st;
    }
    const SBLayout L = sb_layout(jobs, n_jobs, batch);
    if (L.n_tiles > (int64_t)INT32_MAX)
        return fail(BPW_E_UNSUPPORTED, "too many tiles for one launch");
    const size_t need = bpw_gemm_small_batch_workspace_bytes(jobs, n_jobs, batch);
    if (n_jobs > 0 && need > ws_len) return fail(BPW_E_SIZE, "workspace %zu bytes < required %zu", ws_len, need);
    if (n_jobs > 0 && !d_ws) return fail(BPW_E_INVAL, "d_ws is NULL");
    if (((uintptr_t)d_ws & (kAlign - 1)) != 0) return fail(BPW_E_INVAL, "d_ws must be 256-byte aligned");
    bpw_status st = check_device();
    if (st) return st;
    auto *plan = new (std::nothrow) bpw_sb_plan;
    if (!plan) return fail(BPW_E_INVAL, "out of host memory");
    int dev = 0;
    (void)hipGetDevice(&dev);
    uint8_t *ws = static_cast<uint8_t *>(d_ws);
    plan->device = dev;
    plan->jobs = reinterpret_cast<const bpw::SmallBatchArgs *>(ws + L.jobs_off);
    plan->tiles = reinterpret_cast<const bpw::SBTile *>(ws + L.tiles_off);
    plan->n_tiles = L.n_tiles;
    plan->gemv = nullptr;
    plan->tok_jobs = nullptr;
    plan->tok_tiles = nullptr;
    plan->n_tok_tiles = 0;
    plan->nt = 0;
    if (n_jobs == 0 || L.n_tiles == 0) {
        *out = plan;
        return BPW_OK;
    }
    // The token kernel only when pinned: measured on the decode-step set (three HBM copies in
    // rotation) it takes 107.6 us at B = 2 and 142.8 at B = 3, each token adding ~35 us of select work
    // and plane reads, against 102.7 and 107.4 on the matrix cores, whose time barely grows with B.
    if (kernel == BPW_KERNEL_BITSERIAL && batch > 1) {
        // each beat streamed once and reduced against every token's planes on the VALU
        const SBLayout T = tok_layout(jobs, n_jobs);
        std::vector<uint8_t> host(T.total, 0);
        auto *hj = reinterpret_cast<bpw::TokJob *>(host.data() + T.jobs_off);
        auto *hb = reinterpret_cast<bpw::Tile *>(host.data() + T.tiles_off);
        int64_t t = 0;
        for (int32_t i = 0; i < n_jobs; ++i) {
            const bpw_sb_job &j = jobs[i];
            bpw::TokJob d{};
            d.planes = static_cast<const uint8_t *>(j.m.d_planes);
            d.X = j.d_X;
            d.out_i32 = j.d_out_i32;
            d.out_f32 = j.d_out_f32;
            d.ldx = j.ldx;
            d.plane_bytes = (uint32_t)((uint64_t)j.m.rows * (uint64_t)j.m.bpr * 16u);
            d.rows = (int32_t)j.m.rows;
            d.bpr = (int32_t)j.m.bpr;
            d.w_scale = j.m.w_scale;
            for (int32_t k = 0; k < batch; ++k) d.x_scales[k] = j.x_scales[k];
            hj[i] = d;
            const Geometry g = geometry_for(j.m.bpr);
            const int64_t U = units_of(j.m.rows, g), w = tok_tile_units(g);
            for (int64_t u = 0; u < U; u += w) hb[t++] = bpw::tile_of(i, u, std::min(U, u + w));
        }
        const int xccs = device_xcds();
        if (xccs > kMaxXcds) {
            delete plan;
            return fail(BPW_E_UNSUPPORTED, "device has %d XCDs; the tile table is sized for %lld", xccs,
                        (long long)kMaxXcds);
        }
        const double share = t < 2 * (int64_t)device_cus() ? 1.0 : kTailShare;
        plan->n_tok_tiles = xcd_runs(hb, t, xccs, share);
        plan->tok_jobs = reinterpret_cast<const bpw::TokJob *>(ws + T.jobs_off);
        plan->tok_tiles = reinterpret_cast<const bpw::Tile *>(ws + T.tiles_off);
        plan->nt = batch;
        hipStream_t s = reinterpret_cast<hipStream_t>(stream);
        st = hip_status(hipMemcpyAsync(d_ws, host.data(), T.total, hipMemcpyHostToDevice, s), "hipMemcpyAsync");
        if (!st) st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize");
        if (st) {
            delete plan;
            return st;
        }
        *out = plan;
        return BPW_OK;
    }
    if (batch == 1 && kernel != BPW_KERNEL_MFMA) {
        // one token: the bit-serial batch-1 GEMV streams the planes without decoding them (measured on
        // the decode-step set: 81.7 us against 148 us on the matrix cores)
        const std::vector<bpw_gemv_job> g = sb_as_gemv(jobs, n_jobs);
        st = create_plan(g.data(), n_jobs, nullptr, 0, BPW_KERNEL_BITSERIAL, d_ws, ws_len, stream, &plan->gemv);
        if (st) {
            delete plan;
            return st;
        }
        *out = plan;
        return BPW_OK;
    }
    std::vector<uint8_t> host(L.total, 0);
    auto *hj = reinterpret_cast<bpw::SmallBatchArgs *>(host.data() + L.jobs_off);
    auto *ht = reinterpret_cast<bpw::SBTile *>(host.data() + L.tiles_off);
    const int32_t groups = (batch + 15) / 16;
    int64_t t = 0;
    for (int32_t i = 0; i < n_jobs; ++i) {
        const bpw_sb_job &j = jobs[i];
        hj[i] = small_batch_args(&j.m, j.d_X, batch, j.ldx, j.x_scales, j.d_out_i32, j.d_out_f32);
        for (int64_t r = 0; r < sb_job_tiles(j); ++r)
            for (int32_t gq = 0; gq < groups; ++gq) ht[t++] = bpw::SBTile{i, (int32_t)r, gq, 1};
    }
    const int xccs = device_xcds();
    if (xccs > kMaxXcds) {
        delete plan;
        return fail(BPW_E_UNSUPPORTED, "device has %d XCDs; the tile table is sized for %lld", xccs,
                    (long long)kMaxXcds);
    }
    plan->n_tiles = sb_cost_runs(ht, t, xccs, jobs, sb_tile_bound(t));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    st = hip_status(hipMemcpyAsync(d_ws, host.data(), L.total, hipMemcpyHostToDevice, s), "hipMemcpyAsync");
    if (!st) st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize");
    if (st) {
        delete plan;
        return st;
    }
    *out = plan;
    return BPW_OK;
}

bpw_status bpw_gemm_small_batch_plan_run(const bpw_sb_plan *plan, void *stream) {
    if (!plan) return fail(BPW_E_INVAL, "plan is NULL");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
        return fail(BPW_E_INVAL, "plan was created on device %d, current device is %d", plan->device, dev);
    bpw_status st = check_device();
    if (st) return st;
    if (plan->gemv) return bpw_gemv_plan_run(plan->gemv, stream);
    if (plan->n_tok_tiles > 0)
        return hip_status(bpw::launch_gemv_tokens(plan->tok_jobs, plan->tok_tiles, (int32_t)plan->n_tok_tiles, plan->nt,
                                                  stream),
                          "grouped small batch (bit-serial tokens) launch");
    return hip_status(bpw::launch_gemm_small_batch_grouped(plan->jobs, plan->tiles, (int32_t)plan->n_tiles, stream),
                      "grouped small batch launch");
}

void bpw_gemm_small_batch_plan_free(bpw_sb_plan *plan) {
    if (!plan) return;
    bpw_gemv_plan_free(plan->gemv);
    delete plan;
}

bpw_status bpw_dense_head_gemv(const uint16_t *d_w_bf16, int64_t rows, int64_t cols, const uint16_t *d_x_bf16,
                               float *d_y, void *stream) {
    if (rows < 0 || cols < 0) return fail(BPW_E_INVAL, "bad shape");
    if (rows == 0) return check_device();
    if (!d_w_bf16 || !d_x_bf16 || !d_y) return fail(BPW_E_INVAL, "dense head: NULL argument");
    if (cols % 8 != 0) return fail(BPW_E_UNSUPPORTED, "dense head: cols %lld is not a multiple of 8", (long long)cols);
    if (((uintptr_t)d_w_bf16 & 15u) || ((uintptr_t)d_x_bf16 & 15u))
        return fail(BPW_E_INVAL, "dense head: W and x must be 16-byte aligned");
    bpw_status st = check_device();
    if (st) return st;
    return hip_status(bpw::launch_dense_head(d_w_bf16, rows, cols, d_x_bf16, d_y, stream), "dense head launch");
}

bpw_status bpw_stream_read_probe_shape(const void *d_buf, size_t len, uint32_t *d_sink, int32_t shape,
                                       void *stream) {
    if (!d_buf || !d_sink || (len % 16) || ((uintptr_t)d_buf & 15u))
        return fail(BPW_E_INVAL, "probe: buffer must be non-NULL, 16-byte aligned, len %% 16 == 0");
    if (shape < 0 || shape >= bpw::kProbeShapes)
        return fail(BPW_E_INVAL, "probe: shape %d is not one of 0 .. %d", (int)shape, (int)bpw::kProbeShapes - 1);
    if (len > ((size_t)1 << 40)) return fail(BPW_E_INVAL, "probe: len above 2^40 bytes");
    bpw_status st = check_device();
    if (st) return st;
    return hip_status(bpw::launch_probe(d_buf, len, d_sink, shape, stream), "probe launch");
}

bpw_status bpw_stream_read_probe(const void *d_buf, size_t len, uint32_t *d_sink, void *stream) {
    return bpw_stream_read_probe_shape(d_buf, len, d_sink, 0, stream);
}

bpw_status bpw_cache_flush(void *d_buf, size_t len, void *stream) {
    if (!d_buf || (len % 16) || ((uintptr_t)d_buf & 15u))
        return fail(BPW_E_INVAL, "flush: buffer must be non-NULL, 16-byte aligned, len %% 16 == 0");
    bpw_status st = check_device();
    if (st) return st;
    return hip_status(bpw::launch_flush(d_buf, len, stream), "flush launch");
}

}  // extern "C"

namespace bpw {
uint64_t seal_words(const uint64_t *w, int n) {
    uint64_t h = seal_key();
    for (int i = 0; i < n; ++i) h = mix64(h ^ w[i]);
    return h;
}
int host_check_device() { return check_device(); }
int host_xcds() { return device_xcds(); }
void host_xcd_layout(Tile *tiles, int64_t n) { xcd_contiguous(tiles, n, device_xcds()); }
const uint8_t *host_mat_view(const ::bpw_host_mat *m, int64_t *rows, int64_t *cols, float *w_scale) {
    *rows = m->rows;
    *cols = m->cols;
    *w_scale = m->w_scale;
    return m->planes;
}
}  // namespace bpw


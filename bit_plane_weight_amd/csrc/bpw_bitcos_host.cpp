// bpw_bitcos_host.cpp - host side of the BITCOS layout: packing (from int8 trits or from validated
// .trit planes), upload and the grouped batch-1 GEMV plan. See include/bpw.h for the contract.
//
// Passage followed: "BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits", "A bitmap and
// a sign" (one presence bit per weight, one sign bit per nonzero in column order, set for -1). The
// page leaves the blocking open; the row form here gives every row its own run of sign words, so a
// workgroup can start any row without scanning the rows before it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/bpw.h"
#include "bpw_internal.h"

struct bpw_bitcos_host {
    std::vector<uint64_t> presence;   // rows * bpr
    std::vector<uint32_t> signs;      // row_start[rows] words
    std::vector<uint32_t> row_start;  // rows + 1
    int64_t rows = 0, cols = 0, bpr = 0, nnz = 0;
    float w_scale = 1.0f;
};

struct bpw_bitcos_plan {
    int device;
    const bpw::BitcosJob *jobs;
    const bpw::Tile *tiles;
    int64_t n_tiles;
};

namespace {

bpw_status fail(bpw_status code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
bpw_status fail(bpw_status code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    bpw::record_error(buf);
    return code;
}

bpw_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return BPW_OK;
    return fail(BPW_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
constexpr int64_t kMaxCols = 64 * bpw::kXPassBlocks;  // one LDS pass of activation planes
constexpr int64_t kSignPadWords = 4;                 // a 16-byte sign window read at the last word stays in range
constexpr uint64_t kMaxRange = 0xFFFFFFF0ull;        // the kernel's buffer offsets are 32-bit

inline size_t align_up(size_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct DevLayout {
    size_t presence_bytes, row_start_off, row_start_bytes, signs_off, sign_bytes, total;
};

DevLayout dev_layout(int64_t rows, int64_t bpr, int64_t sign_words) {
    DevLayout L{};
    L.presence_bytes = (size_t)rows * (size_t)bpr * 8u;
    L.row_start_off = align_up(L.presence_bytes);
    L.row_start_bytes = (size_t)(rows + 1) * 4u;
    L.signs_off = L.row_start_off + align_up(L.row_start_bytes);
    L.sign_bytes = (size_t)(sign_words + kSignPadWords) * 4u;
    L.total = L.signs_off + align_up(L.sign_bytes);
    return L;
}

// Shape limits of the kernel: cols within one LDS pass, rows addressable as int32, each of the three
// device arrays within 32-bit byte offsets. sign_words < 0: only the first two (before packing).
bpw_status check_shape(int64_t rows, int64_t cols, int64_t sign_words) {
    if (rows < 0 || cols < 0) return fail(BPW_E_INVAL, "negative shape %lld x %lld", (long long)rows, (long long)cols);
    if (cols > kMaxCols)
        return fail(BPW_E_UNSUPPORTED, "%lld columns; the BITCOS kernel serves at most %lld", (long long)cols,
                    (long long)kMaxCols);
    const int64_t bpr = (cols + 63) / 64;
    if (rows > (int64_t)INT32_MAX || (uint64_t)rows * (uint64_t)bpr * 8u >= kMaxRange ||
        (uint64_t)(rows + 1) * 4u >= kMaxRange)
        return fail(BPW_E_UNSUPPORTED, "%lld rows exceed the 32-bit offsets of one matrix", (long long)rows);
    if (sign_words >= 0 && (uint64_t)(sign_words + kSignPadWords) * 4u >= kMaxRange)
        return fail(BPW_E_UNSUPPORTED, "%lld sign words exceed the 32-bit offsets of one matrix",
                    (long long)sign_words);
    return BPW_OK;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }

// Append one row given as its presence and neg (-1) words; the row's signs start a fresh word.
void append_row(bpw_bitcos_host &h, const uint64_t *pres, const uint64_t *neg) {
    h.row_start.push_back((uint32_t)h.signs.size());
    uint64_t k = 0;  // nonzeros of the row so far
    uint32_t cur = 0;
    for (int64_t b = 0; b < h.bpr; ++b) {
        h.presence.push_back(pres[b]);
        uint64_t p = pres[b];
        while (p) {
            const int c = __builtin_ctzll(p);
            p &= p - 1;
            if ((neg[b] >> c) & 1u) cur |= 1u << (k & 31);
            if ((++k & 31) == 0) {
                h.signs.push_back(cur);
                cur = 0;
            }
        }
    }
    if (k & 31) h.signs.push_back(cur);
    h.nnz += (int64_t)k;
}

bpw_status finish(bpw_bitcos_host *h, bpw_bitcos_host **out) {
    h->row_start.push_back((uint32_t)h->signs.size());
    bpw_status st = check_shape(h->rows, h->cols, (int64_t)h->signs.size());
    if (st) {
        delete h;
        return st;
    }
    *out = h;
    return BPW_OK;
}

}  // namespace

extern "C" {

bpw_status bpw_bitcos_pack_i8(const int8_t *w, int64_t rows, int64_t cols, float w_scale, bpw_bitcos_host **out,
                              bpw_err *err) {
    if (err) *err = bpw_err{BPW_OK, -1, -1, -1};
    if (!out) return fail(BPW_E_INVAL, "out is NULL");
    *out = nullptr;
    bpw_status st = check_shape(rows, cols, -1);
    if (st) return st;
    if (rows * cols > 0 && !w) return fail(BPW_E_INVAL, "w is NULL");
    if (!scale_ok(w_scale)) return fail(BPW_E_INVAL, "w_scale must be finite and > 0");
    auto *h = new (std::nothrow) bpw_bitcos_host;
    if (!h) return fail(BPW_E_INVAL, "out of host memory");
    h->rows = rows;
    h->cols = cols;
    h->bpr = (cols + 63) / 64;
    h->w_scale = w_scale;
    try {
        h->presence.reserve((size_t)rows * (size_t)h->bpr);
        h->row_start.reserve((size_t)rows + 1);
        std::vector<uint64_t> pres((size_t)h->bpr), neg((size_t)h->bpr);
        for (int64_t r = 0; r < rows; ++r) {
            std::fill(pres.begin(), pres.end(), 0);
            std::fill(neg.begin(), neg.end(), 0);
            const int8_t *row = w + r * cols;
            for (int64_t c = 0; c < cols; ++c) {
                const int8_t v = row[c];
                if (v < -1 || v > 1) {
                    if (err) *err = bpw_err{BPW_E_INVAL, r, c / 64, c};
                    delete h;
                    return fail(BPW_E_INVAL, "w[%lld, %lld] = %d is not in {-1, 0, +1}", (long long)r, (long long)c,
                                (int)v);
                }
                if (v) pres[(size_t)(c >> 6)] |= UINT64_C(1) << (c & 63);
                if (v < 0) neg[(size_t)(c >> 6)] |= UINT64_C(1) << (c & 63);
            }
            append_row(*h, pres.data(), neg.data());
        }
    } catch (const std::bad_alloc &) {
        delete h;
        return fail(BPW_E_INVAL, "out of host memory");
    }
    return finish(h, out);
}

bpw_status bpw_bitcos_from_planes(const bpw_host_mat *m, bpw_bitcos_host **out) {
    if (!out) return fail(BPW_E_INVAL, "out is NULL");
    *out = nullptr;
    if (!m) return fail(BPW_E_INVAL, "matrix is NULL");
    int64_t rows = 0, cols = 0;
    float w_scale = 0.0f;
    const uint8_t *planes = bpw::host_mat_view(m, &rows, &cols, &w_scale);
    bpw_status st = check_shape(rows, cols, -1);
    if (st) return st;
    auto *h = new (std::nothrow) bpw_bitcos_host;
    if (!h) return fail(BPW_E_INVAL, "out of host memory");
    h->rows = rows;
    h->cols = cols;
    h->bpr = (cols + 63) / 64;
    h->w_scale = w_scale;
    try {
        h->presence.reserve((size_t)rows * (size_t)h->bpr);
        h->row_start.reserve((size_t)rows + 1);
        std::vector<uint64_t> pres((size_t)h->bpr), neg((size_t)h->bpr);
        for (int64_t r = 0; r < rows; ++r) {
            // the matrix was validated on load (P1, P2): pos and neg are disjoint, padding is clear
            for (int64_t b = 0; b < h->bpr; ++b) {
                uint64_t pos, ng;
                std::memcpy(&pos, planes + ((size_t)r * (size_t)h->bpr + (size_t)b) * 16u, 8);
                std::memcpy(&ng, planes + ((size_t)r * (size_t)h->bpr + (size_t)b) * 16u + 8u, 8);
                pres[(size_t)b] = pos | ng;
                neg[(size_t)b] = ng;
            }
            append_row(*h, pres.data(), neg.data());
        }
    } catch (const std::bad_alloc &) {
        delete h;
        return fail(BPW_E_INVAL, "out of host memory");
    }
    return finish(h, out);
}

void bpw_bitcos_free(bpw_bitcos_host *h) { delete h; }

bpw_status bpw_bitcos_arrays(const bpw_bitcos_host *h, const uint64_t **presence, const uint32_t **signs,
                             const uint32_t **row_start, int64_t *sign_words, int64_t *nnz) {
    if (!h) return fail(BPW_E_INVAL, "BITCOS matrix is NULL");
    if (presence) *presence = h->presence.data();
    if (signs) *signs = h->signs.data();
    if (row_start) *row_start = h->row_start.data();
    if (sign_words) *sign_words = (int64_t)h->signs.size();
    if (nnz) *nnz = h->nnz;
    return BPW_OK;
}

size_t bpw_bitcos_device_bytes(const bpw_bitcos_host *h) {
    if (!h) return 0;
    return dev_layout(h->rows, h->bpr, (int64_t)h->signs.size()).total;
}

}  // extern "C"

namespace {

uint64_t seal_of(const bpw_dev_bitcos &m) {
    uint32_t sb;
    std::memcpy(&sb, &m.w_scale, 4);
    const uint64_t w[8] = {(uint64_t)(uintptr_t)m.d_base, (uint64_t)m.rows, (uint64_t)m.cols, (uint64_t)m.bpr,
                           (uint64_t)m.sign_words, m.row_start_off, m.signs_off,
                           (uint64_t)sb | ((uint64_t)m.reserved << 32)};
    return bpw::seal_words(w, 8) ^ UINT64_C(0x42495443'4F530001);  // a domain apart from bpw_dev_mat seals
}

bpw_status check_job(const bpw_bitcos_job &j, int32_t i) {
    if (j.m.seal != seal_of(j.m))
        return fail(BPW_E_NOT_VALIDATED, "job %d: BITCOS descriptor was not produced by bpw_bitcos_upload (or was "
                                         "modified)", i);
    if (!j.d_x) return fail(BPW_E_INVAL, "job %d: d_x is NULL", i);
    if (((uintptr_t)j.d_x & 15u) != 0) return fail(BPW_E_INVAL, "job %d: d_x must be 16-byte aligned", i);
    if (j.x_len < j.m.bpr * 64)
        return fail(BPW_E_INVAL, "job %d: x_len %lld < bpr * 64 = %lld", i, (long long)j.x_len,
                    (long long)(j.m.bpr * 64));
    if (!j.d_out_i32) return fail(BPW_E_INVAL, "job %d: d_out_i32 is NULL", i);
    if (!std::isfinite(j.x_scale)) return fail(BPW_E_INVAL, "job %d: x_scale is not finite", i);
    return BPW_OK;
}

// Row-groups of one job: 64 / 2^glog rows each (the rows one wave covers at a time).
inline int64_t job_units(const bpw_dev_bitcos &m) {
    const int64_t unit_rows = 64 >> bpw::bitcos_geometry(m.bpr).glog;
    return (m.rows + unit_rows - 1) / unit_rows;
}

inline int64_t job_tiles(const bpw_bitcos_job &j) {
    return (job_units(j.m) + bpw::kBcTileUnits - 1) / bpw::kBcTileUnits;
}

struct PlanLayout {
    size_t tiles_off, total;
    int64_t n_tiles;
};

PlanLayout plan_layout(const bpw_bitcos_job *jobs, int32_t n) {
    PlanLayout L{};
    for (int32_t i = 0; i < n; ++i) L.n_tiles += job_tiles(jobs[i]);
    L.tiles_off = align_up(sizeof(bpw::BitcosJob) * (size_t)n);
    L.total = align_up(L.tiles_off + sizeof(bpw::Tile) * (size_t)L.n_tiles);
    return L;
}

}  // namespace

extern "C" {

bpw_status bpw_bitcos_upload(const bpw_bitcos_host *h, void *d_dst, size_t d_len, void *stream, bpw_dev_bitcos *out) {
    if (!h || !out) return fail(BPW_E_INVAL, "NULL matrix or output descriptor");
    std::memset(out, 0, sizeof *out);
    const DevLayout L = dev_layout(h->rows, h->bpr, (int64_t)h->signs.size());
    if (!d_dst) return fail(BPW_E_INVAL, "d_dst is NULL");
    if (d_len < L.total) return fail(BPW_E_SIZE, "d_len %zu < device bytes %zu", d_len, L.total);
    if (((uintptr_t)d_dst & (kAlign - 1)) != 0) return fail(BPW_E_INVAL, "d_dst must be 256-byte aligned");
    bpw_status st = (bpw_status)bpw::host_check_device();
    if (st) return st;
    // one staging image: presence, row_start, signs and the zero padding behind each array
    std::vector<uint8_t> img;
    try {
        img.assign(L.total, 0);
    } catch (const std::bad_alloc &) {
        return fail(BPW_E_INVAL, "out of host memory");
    }
    if (L.presence_bytes) std::memcpy(img.data(), h->presence.data(), L.presence_bytes);
    std::memcpy(img.data() + L.row_start_off, h->row_start.data(), L.row_start_bytes);
    if (!h->signs.empty()) std::memcpy(img.data() + L.signs_off, h->signs.data(), h->signs.size() * 4u);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    st = hip_status(hipMemcpyAsync(d_dst, img.data(), L.total, hipMemcpyHostToDevice, s), "hipMemcpyAsync");
    if (!st) st = hip_status(hipStreamSynchronize(s), "hipStreamSynchronize");
    if (st) return st;
    out->d_base = d_dst;
    out->rows = h->rows;
    out->cols = h->cols;
    out->bpr = h->bpr;
    out->sign_words = (int64_t)h->signs.size();
    out->row_start_off = L.row_start_off;
    out->signs_off = L.signs_off;
    out->w_scale = h->w_scale;
    out->reserved = 0;
    out->seal = seal_of(*out);
    return BPW_OK;
}

size_t bpw_bitcos_workspace_bytes(const bpw_bitcos_job *jobs, int32_t n_jobs) {
    if (!jobs || n_jobs <= 0) return 0;
    return plan_layout(jobs, n_jobs).total;
}

bpw_status bpw_bitcos_plan_create(const bpw_bitcos_job *jobs, int32_t n_jobs, void *d_ws, size_t ws_len, void *stream,
                                  bpw_bitcos_plan **out) {
    if (!out) return fail(BPW_E_INVAL, "out is NULL");
    *out = nullptr;
    if (n_jobs < 0 || (n_jobs > 0 && !jobs)) return fail(BPW_E_INVAL, "bad job list");
    for (int32_t i = 0; i < n_jobs; ++i) {
        bpw_status st = check_job(jobs[i], i);
        if (st) return st;
    }
    const PlanLayout L = plan_layout(jobs, n_jobs);
    if (L.n_tiles > (int64_t)INT32_MAX) return fail(BPW_E_UNSUPPORTED, "too many tiles for one launch");
    if (n_jobs > 0 && L.total > ws_len) return fail(BPW_E_SIZE, "workspace %zu bytes < required %zu", ws_len, L.total);
    if (n_jobs > 0 && !d_ws) return fail(BPW_E_INVAL, "d_ws is NULL");
    if (((uintptr_t)d_ws & (kAlign - 1)) != 0) return fail(BPW_E_INVAL, "d_ws must be 256-byte aligned");
    bpw_status st = (bpw_status)bpw::host_check_device();
    if (st) return st;
    int dev = 0;
    (void)hipGetDevice(&dev);
    auto *plan = new (std::nothrow) bpw_bitcos_plan;
    if (!plan) return fail(BPW_E_INVAL, "out of host memory");
    uint8_t *ws = static_cast<uint8_t *>(d_ws);
    plan->device = dev;
    plan->jobs = reinterpret_cast<const bpw::BitcosJob *>(ws);
    plan->tiles = reinterpret_cast<const bpw::Tile *>(ws + L.tiles_off);
    plan->n_tiles = L.n_tiles;
    if (L.n_tiles == 0) {
        *out = plan;
        return BPW_OK;
    }
    std::vector<uint8_t> host(L.total, 0);
    auto *hj = reinterpret_cast<bpw::BitcosJob *>(host.data());
    auto *ht = reinterpret_cast<bpw::Tile *>(host.data() + L.tiles_off);
    int64_t t = 0;
    for (int32_t i = 0; i < n_jobs; ++i) {
        const bpw_bitcos_job &j = jobs[i];
        const uint8_t *base = static_cast<const uint8_t *>(j.m.d_base);
        const DevLayout D = dev_layout(j.m.rows, j.m.bpr, j.m.sign_words);
        bpw::BitcosJob d{};
        d.presence = reinterpret_cast<const uint64_t *>(base);
        d.row_start = reinterpret_cast<const uint32_t *>(base + j.m.row_start_off);
        d.signs = reinterpret_cast<const uint32_t *>(base + j.m.signs_off);
        d.x = j.d_x;
        d.out_i32 = j.d_out_i32;
        d.out_f32 = j.d_out_f32;
        d.rows = (int32_t)j.m.rows;
        d.bpr = (int32_t)j.m.bpr;
        d.x_scale = j.x_scale;
        d.w_scale = j.m.w_scale;
        d.presence_bytes = (uint32_t)D.presence_bytes;
        d.row_start_bytes = (uint32_t)D.row_start_bytes;
        d.sign_bytes = (uint32_t)D.sign_bytes;
        hj[i] = d;
        const int64_t U = job_units(j.m);
        for (int64_t u = 0; u < U; u += bpw::kBcTileUnits)
            ht[t++] = bpw::tile_of(i, u, std::min(U, u + bpw::kBcTileUnits));
    }
    bpw::host_xcd_layout(ht, t);
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

bpw_status bpw_bitcos_plan_run(const bpw_bitcos_plan *plan, void *stream) {
    if (!plan) return fail(BPW_E_INVAL, "plan is NULL");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->device)
        return fail(BPW_E_INVAL, "plan was created on device %d, current device is %d", plan->device, dev);
    bpw_status st = (bpw_status)bpw::host_check_device();
    if (st) return st;
    if (plan->n_tiles == 0) return BPW_OK;
    return hip_status((hipError_t)bpw::launch_gemv_bitcos(plan->jobs, plan->tiles, (int32_t)plan->n_tiles, stream),
                      "BITCOS GEMV launch");
}

void bpw_bitcos_plan_free(bpw_bitcos_plan *plan) { delete plan; }

}  // extern "C"

// bpw_trit.cpp - .trit v1 container reader and writer ("The .trit format, version 1": section 2 "File
// layout", 2.1 "Header fields", 2.2 "Tensor record", 2.3 "Ternary payload", 2.4 "Dense payload",
// section 4 "Validation", section 6 "What a reader is allowed to assume"). Host only.
//
// The file is untrusted: every read is bounds-checked against the file length before it happens,
// every size sum is overflow-checked, and every failure is a status with the check's number. Fields
// are read in file order and each is checked as soon as it has been read; a field that would extend
// past the end of the file is check 5. Within a record: name_len, name (and duplicates), dtype,
// ndim, reserved0, reserved1, dims, shape product (9), scale, flags, offset, byte_len, then 14 and
// 15/16. After the table the payload starts at the next multiple of 64 (past the end of the file:
// check 5), then every extent is checked against the payload (12, record order) and against the
// others (13, extents in offset order). tensor_count above 1,048,576 and a name that is not valid
// UTF-8 count as check 7; the padding before the payload is not inspected.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <unordered_set>
#include <vector>
#include <algorithm>

#include "../../include/bpw.h"
#include "bpw_internal.h"

namespace {

constexpr uint32_t kMaxConfig = 16u * 1024u * 1024u;
constexpr uint32_t kMaxTensors = 1048576u;
constexpr uint32_t kMaxName = 1024u;

struct Rec {
    uint64_t name_off;
    uint32_t name_len;
    uint8_t dtype;
    uint8_t ndim;
    uint32_t dims[4];
    float scale;
    uint64_t offset;
    uint64_t byte_len;
};

bpw_status tfail(bpw_trit_err *e, bpw_status code, int check, int64_t offset, int64_t tensor, const char *fmt, ...)
    __attribute__((format(printf, 6, 7)));
bpw_status tfail(bpw_trit_err *e, bpw_status code, int check, int64_t offset, int64_t tensor, const char *fmt, ...) {
    char buf[400];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    char msg[480];
    std::snprintf(msg, sizeof msg, ".trit check %d: %s", check, buf);
    bpw::record_error(msg);
    if (e) {
        e->code = code;
        e->check = check;
        e->offset = offset;
        e->tensor = tensor;
        e->row = e->beat = e->col = -1;
    }
    return code;
}

void clear_err(bpw_trit_err *e) {
    if (e) {
        e->code = BPW_OK;
        e->check = 0;
        e->offset = e->tensor = e->row = e->beat = e->col = -1;
    }
}

// Strict UTF-8 (the well-formed byte sequences of the Unicode standard: no overlong forms, no
// surrogates, nothing above U+10FFFF).
bool utf8_ok(const uint8_t *p, size_t n) {
    size_t i = 0;
    while (i < n) {
        const uint8_t c = p[i];
        if (c < 0x80) {
            ++i;
            continue;
        }
        size_t len;
        uint8_t lo = 0x80, hi = 0xBF;
        if (c >= 0xC2 && c <= 0xDF) {
            len = 2;
        } else if (c >= 0xE0 && c <= 0xEF) {
            len = 3;
            if (c == 0xE0) lo = 0xA0;
            if (c == 0xED) hi = 0x9F;
        } else if (c >= 0xF0 && c <= 0xF4) {
            len = 4;
            if (c == 0xF0) lo = 0x90;
            if (c == 0xF4) hi = 0x8F;
        } else {
            return false;
        }
        if (i + len > n) return false;
        if (p[i + 1] < lo || p[i + 1] > hi) return false;
        for (size_t k = 2; k < len; ++k)
            if (p[i + k] < 0x80 || p[i + k] > 0xBF) return false;
        i += len;
    }
    return true;
}

// Sequential little-endian reads that refuse to pass the end of the file.
struct Cursor {
    const uint8_t *b;
    size_t n, pos;
    bool take(size_t k) {
        if (k > n - pos) return false;
        pos += k;
        return true;
    }
    template <class T>
    bool get(T &v) {
        if (sizeof(T) > n - pos) return false;
        std::memcpy(&v, b + pos, sizeof(T));  // hosts that run ROCm are little-endian, as the format is
        pos += sizeof(T);
        return true;
    }
};

bool mul_ok(uint64_t a, uint64_t b, uint64_t &r) { return !__builtin_mul_overflow(a, b, &r); }

}  // namespace

struct bpw_trit_file {
    const uint8_t *bytes;
    size_t len;
    uint64_t payload_start;
    uint64_t stored_hash;
    uint64_t config_off;
    uint32_t config_len;
    std::vector<Rec> recs;
};

extern "C" {

uint64_t bpw_fnv1a64(const uint8_t *data, size_t len) {
    uint64_t h = 0xCBF29CE484222325ull;  // FNV-1a 64-bit offset basis
    for (size_t i = 0; i < len; ++i) {
        h ^= data[i];
        h *= 0x100000001B3ull;  // FNV 64-bit prime
    }
    return h;
}

bpw_status bpw_trit_open(const uint8_t *bytes, size_t len, bpw_trit_file **out, bpw_trit_err *err) {
    clear_err(err);
    if (!out) return tfail(err, BPW_E_INVAL, 0, -1, -1, "out is NULL");
    *out = nullptr;
    if (!bytes && len) return tfail(err, BPW_E_INVAL, 0, -1, -1, "bytes is NULL");
    static const uint8_t kEmpty[1] = {0};
    Cursor c{bytes ? bytes : kEmpty, bytes ? len : 0, 0};
    auto trunc = [&](const char *what) {
        return tfail(err, BPW_E_FORMAT, 5, (int64_t)c.pos, -1, "truncated: %s runs past the end of the file", what);
    };
    uint32_t u32 = 0;
    if (c.n < 4) return trunc("magic");
    if (std::memcmp(c.b, "TRIT", 4) != 0)
        return tfail(err, BPW_E_FORMAT, 1, 0, -1, "not a .trit container (the first four bytes are not TRIT)");
    c.pos = 4;
    size_t at = c.pos;
    if (!c.get(u32)) return trunc("version");
    if (u32 == 0)
        return tfail(err, BPW_E_FORMAT, 2, (int64_t)at, -1,
                     "version 0 (interleaved 2-bit codes) is not read; convert the source checkpoint to version 1");
    if (u32 > 1) return tfail(err, BPW_E_FORMAT, 3, (int64_t)at, -1, "version %u is not supported", u32);
    at = c.pos;
    if (!c.get(u32)) return trunc("header_flags");
    if (u32 != 0) return tfail(err, BPW_E_FORMAT, 4, (int64_t)at, -1, "unknown header flags 0x%x", u32);
    uint64_t hash = 0;
    if (!c.get(hash)) return trunc("payload_hash");
    at = c.pos;
    uint32_t config_len = 0;
    if (!c.get(config_len)) return trunc("config_len");
    if (config_len > kMaxConfig)
        return tfail(err, BPW_E_FORMAT, 6, (int64_t)at, -1, "config_len %u exceeds 16 MiB", config_len);
    const uint64_t config_off = c.pos;
    if (!c.take(config_len)) return trunc("config");
    if (!utf8_ok(c.b + config_off, config_len))
        return tfail(err, BPW_E_FORMAT, 6, (int64_t)config_off, -1, "config is not valid UTF-8");
    at = c.pos;
    uint32_t count = 0;
    if (!c.get(count)) return trunc("tensor_count");
    if (count > kMaxTensors)
        return tfail(err, BPW_E_FORMAT, 7, (int64_t)at, -1, "tensor_count %u exceeds 1048576", count);

    auto *f = new (std::nothrow) bpw_trit_file;
    if (!f) return tfail(err, BPW_E_INVAL, 0, -1, -1, "out of host memory");
    f->bytes = c.b;
    f->len = c.n;
    f->stored_hash = hash;
    f->config_off = config_off;
    f->config_len = config_len;
    std::unordered_set<std::string> names;
    bpw_status st = BPW_OK;
    auto bail = [&](bpw_status s) {
        delete f;
        return s;
    };
    try {
        f->recs.reserve(std::min<uint32_t>(count, 65536u));
        names.reserve(std::min<uint32_t>(count, 65536u));
        for (uint32_t i = 0; i < count; ++i) {
            const int64_t ti = (int64_t)i;
            Rec r{};
            at = c.pos;
            uint16_t name_len = 0;
            if (!c.get(name_len)) return bail(trunc("name_len"));
            if (name_len == 0 || name_len > kMaxName)
                return bail(tfail(err, BPW_E_FORMAT, 7, (int64_t)at, ti, "tensor %u: name_len %u outside 1..1024", i,
                                  (unsigned)name_len));
            r.name_off = c.pos;
            r.name_len = name_len;
            if (!c.take(name_len)) return bail(trunc("tensor name"));
            if (!utf8_ok(c.b + r.name_off, name_len))
                return bail(tfail(err, BPW_E_FORMAT, 7, (int64_t)r.name_off, ti, "tensor %u: name is not valid UTF-8", i));
            if (!names.emplace(reinterpret_cast<const char *>(c.b + r.name_off), name_len).second)
                return bail(tfail(err, BPW_E_FORMAT, 7, (int64_t)r.name_off, ti, "tensor %u: duplicate name", i));
            at = c.pos;
            if (!c.get(r.dtype)) return bail(trunc("dtype"));
            if (r.dtype > 2)
                return bail(tfail(err, BPW_E_FORMAT, 8, (int64_t)at, ti, "tensor %u: unknown dtype %u", i,
                                  (unsigned)r.dtype));
            at = c.pos;
            if (!c.get(r.ndim)) return bail(trunc("ndim"));
            if (r.ndim < 1 || r.ndim > 4)
                return bail(tfail(err, BPW_E_FORMAT, 8, (int64_t)at, ti, "tensor %u: ndim %u outside 1..4", i,
                                  (unsigned)r.ndim));
            for (int k = 0; k < 2; ++k) {
                at = c.pos;
                uint8_t rsv = 0;
                if (!c.get(rsv)) return bail(trunc("reserved byte"));
                if (rsv != 0)
                    return bail(tfail(err, BPW_E_FORMAT, 8, (int64_t)at, ti, "tensor %u: reserved%d is %u", i, k,
                                      (unsigned)rsv));
            }
            at = c.pos;
            uint64_t prod = 1;
            bool overflow = false;
            for (int k = 0; k < r.ndim; ++k) {
                if (!c.get(r.dims[k])) return bail(trunc("dims"));
                overflow |= !mul_ok(prod, r.dims[k], prod);
            }
            if (overflow)
                return bail(tfail(err, BPW_E_FORMAT, 9, (int64_t)at, ti, "tensor %u: shape product overflows", i));
            at = c.pos;
            if (!c.get(r.scale)) return bail(trunc("scale"));
            if (!std::isfinite(r.scale) || !(r.scale > 0.0f))
                return bail(tfail(err, BPW_E_FORMAT, 10, (int64_t)at, ti, "tensor %u: scale %g is not finite and > 0", i,
                                  (double)r.scale));
            at = c.pos;
            if (!c.get(u32)) return bail(trunc("flags"));
            if (u32 != 0)
                return bail(tfail(err, BPW_E_FORMAT, 8, (int64_t)at, ti, "tensor %u: unknown flags 0x%x", i, u32));
            at = c.pos;
            if (!c.get(r.offset)) return bail(trunc("offset"));
            if (r.offset % 64 != 0)
                return bail(tfail(err, BPW_E_FORMAT, 11, (int64_t)at, ti, "tensor %u: offset %llu is not a multiple of 64",
                                  i, (unsigned long long)r.offset));
            at = c.pos;
            if (!c.get(r.byte_len)) return bail(trunc("byte_len"));
            uint64_t expect = 0;
            if (r.dtype == BPW_TRIT_TERNARY) {
                if (r.ndim != 2)
                    return bail(tfail(err, BPW_E_FORMAT, 14, (int64_t)at, ti, "tensor %u: ternary with ndim %u", i,
                                      (unsigned)r.ndim));
                const uint64_t bpr = ((uint64_t)r.dims[1] + 63) / 64;
                if (!mul_ok((uint64_t)r.dims[0], bpr, expect) || !mul_ok(expect, 16, expect))
                    return bail(tfail(err, BPW_E_FORMAT, 9, (int64_t)at, ti, "tensor %u: byte count overflows", i));
                if (r.byte_len != expect)
                    return bail(tfail(err, BPW_E_FORMAT, 15, (int64_t)at, ti,
                                      "tensor %u: byte_len %llu != rows * beats_per_row * 16 = %llu", i,
                                      (unsigned long long)r.byte_len, (unsigned long long)expect));
            } else {
                if (!mul_ok(prod, r.dtype == BPW_TRIT_F32 ? 4 : 2, expect))
                    return bail(tfail(err, BPW_E_FORMAT, 9, (int64_t)at, ti, "tensor %u: byte count overflows", i));
                if (r.byte_len != expect)
                    return bail(tfail(err, BPW_E_FORMAT, 16, (int64_t)at, ti,
                                      "tensor %u: byte_len %llu != elements * element size = %llu", i,
                                      (unsigned long long)r.byte_len, (unsigned long long)expect));
            }
            f->recs.push_back(r);
        }
        const uint64_t start = ((uint64_t)c.pos + 63) / 64 * 64;
        if (start > c.n) return bail(tfail(err, BPW_E_FORMAT, 5, (int64_t)c.pos, -1, "truncated: no payload start"));
        f->payload_start = start;
        const uint64_t payload_len = c.n - start;
        for (uint32_t i = 0; i < count; ++i) {
            const Rec &r = f->recs[i];
            if (r.offset > payload_len || r.byte_len > payload_len - r.offset)
                return bail(tfail(err, BPW_E_FORMAT, 12, -1, (int64_t)i, "tensor %u: extent runs past the payload", i));
        }
        std::vector<uint32_t> order(count);
        for (uint32_t i = 0; i < count; ++i) order[i] = i;
        std::sort(order.begin(), order.end(), [&](uint32_t a, uint32_t b) {
            return f->recs[a].offset != f->recs[b].offset ? f->recs[a].offset < f->recs[b].offset : a < b;
        });
        uint64_t end = 0;
        bool any = false;
        for (const uint32_t i : order) {
            const Rec &r = f->recs[i];
            if (r.byte_len == 0) continue;
            if (any && r.offset < end)
                return bail(tfail(err, BPW_E_FORMAT, 13, -1, (int64_t)i, "tensor %u overlaps another tensor", i));
            end = r.offset + r.byte_len;
            any = true;
        }
    } catch (const std::bad_alloc &) {
        return bail(tfail(err, BPW_E_INVAL, 0, -1, -1, "out of host memory"));
    }
    (void)st;
    *out = f;
    return BPW_OK;
}

bpw_status bpw_trit_verify(const bpw_trit_file *f, int32_t check_hash, bpw_trit_err *err) {
    clear_err(err);
    if (!f) return tfail(err, BPW_E_INVAL, 0, -1, -1, "file is NULL");
    for (size_t i = 0; i < f->recs.size(); ++i) {
        const Rec &r = f->recs[i];
        if (r.dtype != BPW_TRIT_TERNARY) continue;
        const uint64_t rows = r.dims[0], cols = r.dims[1], bpr = (cols + 63) / 64;
        const uint64_t tail = (cols % 64 == 0) ? ~0ull : ((1ull << (cols % 64)) - 1ull);
        const uint8_t *p = f->bytes + f->payload_start + r.offset;
        for (uint64_t row = 0; row < rows; ++row) {
            for (uint64_t b = 0; b < bpr; ++b) {
                uint64_t pos, neg;
                std::memcpy(&pos, p + (row * bpr + b) * 16, 8);
                std::memcpy(&neg, p + (row * bpr + b) * 16 + 8, 8);
                const uint64_t both = pos & neg;
                const uint64_t pad = b + 1 == bpr ? (pos | neg) & ~tail : 0;
                if (both || pad) {
                    const bool p1 = both != 0;
                    const uint64_t bits = p1 ? both : pad;
                    bpw_status s = tfail(err, p1 ? BPW_E_P1_BOTH_BITS : BPW_E_P2_PADDING, p1 ? 17 : 18,
                                         (int64_t)(f->payload_start + r.offset + (row * bpr + b) * 16), (int64_t)i,
                                         "tensor %zu: %s at row %llu, beat %llu, column %llu", i,
                                         p1 ? "a weight is both +1 and -1" : "a padding bit is set",
                                         (unsigned long long)row, (unsigned long long)b,
                                         (unsigned long long)(64 * b + (uint64_t)__builtin_ctzll(bits)));
                    if (err) {
                        err->row = (int64_t)row;
                        err->beat = (int64_t)b;
                        err->col = (int64_t)(64 * b + (uint64_t)__builtin_ctzll(bits));
                    }
                    return s;
                }
            }
        }
    }
    if (check_hash && f->stored_hash != 0) {
        const uint64_t h = bpw_fnv1a64(f->bytes + f->payload_start, f->len - f->payload_start);
        if (h != f->stored_hash)
            return tfail(err, BPW_E_FORMAT, 19, 12, -1, "payload hash 0x%016llx != stored 0x%016llx",
                         (unsigned long long)h, (unsigned long long)f->stored_hash);
    }
    return BPW_OK;
}

void bpw_trit_close(bpw_trit_file *f) { delete f; }

int64_t bpw_trit_tensor_count(const bpw_trit_file *f) { return f ? (int64_t)f->recs.size() : -1; }

bpw_status bpw_trit_tensor_info(const bpw_trit_file *f, int64_t index, bpw_trit_tensor *out) {
    if (!f || !out) return tfail(nullptr, BPW_E_INVAL, 0, -1, -1, "NULL argument");
    if (index < 0 || index >= (int64_t)f->recs.size())
        return tfail(nullptr, BPW_E_INVAL, 0, -1, index, "tensor index %lld out of range", (long long)index);
    const Rec &r = f->recs[(size_t)index];
    *out = bpw_trit_tensor{};
    out->name = reinterpret_cast<const char *>(f->bytes + r.name_off);
    out->name_len = r.name_len;
    out->dtype = r.dtype;
    out->ndim = r.ndim;
    for (int k = 0; k < r.ndim; ++k) out->dims[k] = r.dims[k];
    out->scale = r.scale;
    out->offset = r.offset;
    out->byte_len = r.byte_len;
    out->data = f->bytes + f->payload_start + r.offset;
    return BPW_OK;
}

int64_t bpw_trit_find(const bpw_trit_file *f, const char *name, size_t name_len) {
    if (!f || !name) return -1;
    for (size_t i = 0; i < f->recs.size(); ++i) {
        const Rec &r = f->recs[i];
        if (r.name_len == name_len && std::memcmp(f->bytes + r.name_off, name, name_len) == 0) return (int64_t)i;
    }
    return -1;
}

bpw_status bpw_trit_config(const bpw_trit_file *f, const char **json, size_t *len) {
    if (!f || !json || !len) return tfail(nullptr, BPW_E_INVAL, 0, -1, -1, "NULL argument");
    *json = reinterpret_cast<const char *>(f->bytes + f->config_off);
    *len = f->config_len;
    return BPW_OK;
}

uint64_t bpw_trit_stored_hash(const bpw_trit_file *f) { return f ? f->stored_hash : 0; }

bpw_status bpw_trit_load(const bpw_trit_file *f, int64_t index, bpw_host_mat **out, bpw_err *err) {
    if (out) *out = nullptr;
    if (!f || !out) return tfail(nullptr, BPW_E_INVAL, 0, -1, -1, "NULL argument");
    if (index < 0 || index >= (int64_t)f->recs.size())
        return tfail(nullptr, BPW_E_INVAL, 0, -1, index, "tensor index %lld out of range", (long long)index);
    const Rec &r = f->recs[(size_t)index];
    if (r.dtype != BPW_TRIT_TERNARY)
        return tfail(nullptr, BPW_E_INVAL, 0, -1, index, "tensor %lld is not ternary", (long long)index);
    return bpw_load(f->bytes + f->payload_start + r.offset, (size_t)r.byte_len, (int64_t)r.dims[0],
                    (int64_t)r.dims[1], r.scale, out, err);
}

}  // extern "C"

// ------------------------------------------------------------------------------------------
// Writer. Deterministic: records sorted by name bytewise (section 2.2 asks for sorted names so that
// conversions are byte-identical), payloads packed in that order at multiples of 64, the file ending
// with the last tensor's bytes. Every input is checked first, each failure numbered by the reader
// check it would trip, so that what this writes always opens and verifies.

namespace {

constexpr uint64_t align64(uint64_t v) { return (v + 63) / 64 * 64; }

struct WriteLayout {
    std::vector<uint32_t> order;    // caller indices in record order
    std::vector<uint64_t> offsets;  // payload offset of each tensor, by caller index
    uint64_t payload_start = 0;
    uint64_t payload_len = 0;       // offset of the last record plus its byte_len
};

bool name_less(const bpw_trit_tensor_in &a, const bpw_trit_tensor_in &b) {
    return std::lexicographical_compare(reinterpret_cast<const uint8_t *>(a.name),
                                        reinterpret_cast<const uint8_t *>(a.name) + a.name_len,
                                        reinterpret_cast<const uint8_t *>(b.name),
                                        reinterpret_cast<const uint8_t *>(b.name) + b.name_len);
}

// The field checks of one tensor, in record order.
bpw_status check_tensor_in(const bpw_trit_tensor_in &t, int64_t i, bpw_trit_err *err) {
    if (!t.name || t.name_len < 1 || t.name_len > (int64_t)kMaxName)
        return tfail(err, BPW_E_FORMAT, 7, -1, i, "tensor %lld: name_len %lld outside 1..1024 (or name NULL)",
                     (long long)i, (long long)t.name_len);
    if (!utf8_ok(reinterpret_cast<const uint8_t *>(t.name), (size_t)t.name_len))
        return tfail(err, BPW_E_FORMAT, 7, -1, i, "tensor %lld: name is not valid UTF-8", (long long)i);
    if (t.dtype < 0 || t.dtype > 2)
        return tfail(err, BPW_E_FORMAT, 8, -1, i, "tensor %lld: unknown dtype %d", (long long)i, (int)t.dtype);
    if (t.ndim < 1 || t.ndim > 4)
        return tfail(err, BPW_E_FORMAT, 8, -1, i, "tensor %lld: ndim %d outside 1..4", (long long)i, (int)t.ndim);
    if (t.reserved != 0)
        return tfail(err, BPW_E_FORMAT, 8, -1, i, "tensor %lld: reserved is %u", (long long)i, t.reserved);
    uint64_t prod = 1;
    bool overflow = false;
    for (int k = 0; k < t.ndim; ++k) overflow |= !mul_ok(prod, t.dims[k], prod);
    if (overflow) return tfail(err, BPW_E_FORMAT, 9, -1, i, "tensor %lld: shape product overflows", (long long)i);
    if (!std::isfinite(t.scale) || !(t.scale > 0.0f))
        return tfail(err, BPW_E_FORMAT, 10, -1, i, "tensor %lld: scale %g is not finite and > 0", (long long)i,
                     (double)t.scale);
    uint64_t expect = 0;
    if (t.dtype == BPW_TRIT_TERNARY) {
        if (t.ndim != 2)
            return tfail(err, BPW_E_FORMAT, 14, -1, i, "tensor %lld: ternary with ndim %d", (long long)i, (int)t.ndim);
        const uint64_t bpr = ((uint64_t)t.dims[1] + 63) / 64;
        if (!mul_ok((uint64_t)t.dims[0], bpr, expect) || !mul_ok(expect, 16, expect))
            return tfail(err, BPW_E_FORMAT, 9, -1, i, "tensor %lld: byte count overflows", (long long)i);
        if (t.byte_len != expect)
            return tfail(err, BPW_E_FORMAT, 15, -1, i, "tensor %lld: byte_len %llu != rows * beats_per_row * 16 = %llu",
                         (long long)i, (unsigned long long)t.byte_len, (unsigned long long)expect);
    } else {
        if (!mul_ok(prod, t.dtype == BPW_TRIT_F32 ? 4 : 2, expect))
            return tfail(err, BPW_E_FORMAT, 9, -1, i, "tensor %lld: byte count overflows", (long long)i);
        if (t.byte_len != expect)
            return tfail(err, BPW_E_FORMAT, 16, -1, i, "tensor %lld: byte_len %llu != elements * element size = %llu",
                         (long long)i, (unsigned long long)t.byte_len, (unsigned long long)expect);
    }
    if (t.byte_len > 0 && !t.data)
        return tfail(err, BPW_E_INVAL, 0, -1, i, "tensor %lld: data is NULL", (long long)i);
    return BPW_OK;
}

// Checks every tensor and the counts, sorts, and places the payloads. The config's bytes are checked
// by the caller (bpw_trit_write_size sees only their length).
bpw_status write_layout(const bpw_trit_tensor_in *t, int64_t n, size_t config_len, WriteLayout &L, bpw_trit_err *err) {
    if (n < 0 || (n > 0 && !t)) return tfail(err, BPW_E_INVAL, 0, -1, -1, "bad tensor list");
    if (config_len > kMaxConfig)
        return tfail(err, BPW_E_FORMAT, 6, -1, -1, "config_len %zu exceeds 16 MiB", config_len);
    if (n > (int64_t)kMaxTensors)
        return tfail(err, BPW_E_FORMAT, 7, -1, -1, "%lld tensors exceed 1048576", (long long)n);
    uint64_t head = 4 + 4 + 4 + 8 + 4 + (uint64_t)config_len + 4;
    for (int64_t i = 0; i < n; ++i) {
        const bpw_status st = check_tensor_in(t[i], i, err);
        if (st) return st;
        head += 2 + (uint64_t)t[i].name_len + 4 + 4 * (uint64_t)t[i].ndim + 4 + 4 + 8 + 8;
    }
    L.order.resize((size_t)n);
    for (int64_t i = 0; i < n; ++i) L.order[(size_t)i] = (uint32_t)i;
    std::stable_sort(L.order.begin(), L.order.end(), [&](uint32_t a, uint32_t b) { return name_less(t[a], t[b]); });
    for (size_t k = 1; k < L.order.size(); ++k) {
        const bpw_trit_tensor_in &a = t[L.order[k - 1]], &b = t[L.order[k]];
        if (a.name_len == b.name_len && std::memcmp(a.name, b.name, (size_t)a.name_len) == 0)
            return tfail(err, BPW_E_FORMAT, 7, -1, (int64_t)L.order[k], "tensor %u: duplicate name", L.order[k]);
    }
    L.offsets.assign((size_t)n, 0);
    uint64_t off = 0, end = 0;
    for (const uint32_t i : L.order) {
        L.offsets[i] = off;
        if (t[i].byte_len > UINT64_MAX - off - 63)
            return tfail(err, BPW_E_FORMAT, 9, -1, (int64_t)i, "tensor %u: payload size overflows", i);
        end = off + t[i].byte_len;
        off = align64(end);
    }
    L.payload_start = align64(head);
    L.payload_len = end;
    if (L.payload_len > UINT64_MAX - L.payload_start)
        return tfail(err, BPW_E_FORMAT, 9, -1, -1, "container size overflows");
    return BPW_OK;
}

// P1 and P2 of one ternary payload (checks 17 and 18, first offending beat in row-major order).
bpw_status check_planes(const bpw_trit_tensor_in &t, int64_t i, bpw_trit_err *err) {
    const uint64_t rows = t.dims[0], cols = t.dims[1], bpr = (cols + 63) / 64;
    const uint64_t tail = (cols % 64 == 0) ? ~0ull : ((1ull << (cols % 64)) - 1ull);
    for (uint64_t row = 0; row < rows; ++row)
        for (uint64_t b = 0; b < bpr; ++b) {
            uint64_t pos, neg;
            std::memcpy(&pos, t.data + (row * bpr + b) * 16, 8);
            std::memcpy(&neg, t.data + (row * bpr + b) * 16 + 8, 8);
            const uint64_t both = pos & neg;
            const uint64_t pad = b + 1 == bpr ? (pos | neg) & ~tail : 0;
            if (both || pad) {
                const bool p1 = both != 0;
                const int64_t col = (int64_t)(64 * b) + __builtin_ctzll(p1 ? both : pad);
                tfail(err, p1 ? BPW_E_P1_BOTH_BITS : BPW_E_P2_PADDING, p1 ? 17 : 18, -1, i,
                      "tensor %lld: row %llu beat %llu column %lld %s", (long long)i, (unsigned long long)row,
                      (unsigned long long)b, (long long)col, p1 ? "has both bits set" : "has a padding bit set");
                if (err) {
                    err->row = (int64_t)row;
                    err->beat = (int64_t)b;
                    err->col = col;
                }
                return p1 ? BPW_E_P1_BOTH_BITS : BPW_E_P2_PADDING;
            }
        }
    return BPW_OK;
}

template <class T>
uint8_t *put(uint8_t *p, T v) {
    std::memcpy(p, &v, sizeof v);  // little-endian hosts, as the format is
    return p + sizeof v;
}

}  // namespace

extern "C" {

bpw_status bpw_trit_write_size(const bpw_trit_tensor_in *tensors, int64_t n, size_t config_len, uint64_t *bytes,
                               bpw_trit_err *err) {
    clear_err(err);
    if (!bytes) return tfail(err, BPW_E_INVAL, 0, -1, -1, "bytes is NULL");
    *bytes = 0;
    try {
        WriteLayout L;
        const bpw_status st = write_layout(tensors, n, config_len, L, err);
        if (st) return st;
        *bytes = L.payload_start + L.payload_len;
    } catch (const std::bad_alloc &) {
        return tfail(err, BPW_E_INVAL, 0, -1, -1, "out of host memory");
    }
    return BPW_OK;
}

bpw_status bpw_trit_write(const bpw_trit_tensor_in *tensors, int64_t n, const char *config, size_t config_len,
                          int32_t with_hash, uint8_t *out, size_t out_len, uint64_t *written, bpw_trit_err *err) {
    clear_err(err);
    if (!written) return tfail(err, BPW_E_INVAL, 0, -1, -1, "written is NULL");
    *written = 0;
    if (config_len > 0 && !config) return tfail(err, BPW_E_INVAL, 0, -1, -1, "config is NULL");
    if (config_len <= kMaxConfig && !utf8_ok(reinterpret_cast<const uint8_t *>(config), config_len))
        return tfail(err, BPW_E_FORMAT, 6, -1, -1, "config is not valid UTF-8");
    try {
        WriteLayout L;
        bpw_status st = write_layout(tensors, n, config_len, L, err);
        if (st) return st;
        for (int64_t i = 0; i < n; ++i)
            if (tensors[i].dtype == BPW_TRIT_TERNARY && (st = check_planes(tensors[i], i, err)) != BPW_OK) return st;
        const uint64_t total = L.payload_start + L.payload_len;
        if (!out || out_len < total) {
            *written = total;
            return tfail(err, BPW_E_SIZE, 0, -1, -1, "out holds %zu bytes, the container needs %llu", out_len,
                         (unsigned long long)total);
        }
        uint8_t *p = out;
        std::memcpy(p, "TRIT", 4);
        p = put<uint32_t>(p + 4, 1u);           // version
        p = put<uint32_t>(p, 0u);               // header flags
        uint8_t *hash_at = p;
        p = put<uint64_t>(p, 0ull);             // payload hash, below
        p = put<uint32_t>(p, (uint32_t)config_len);
        if (config_len) std::memcpy(p, config, config_len);
        p += config_len;
        p = put<uint32_t>(p, (uint32_t)n);
        for (const uint32_t i : L.order) {
            const bpw_trit_tensor_in &t = tensors[i];
            p = put<uint16_t>(p, (uint16_t)t.name_len);
            std::memcpy(p, t.name, (size_t)t.name_len);
            p += t.name_len;
            p = put<uint8_t>(p, (uint8_t)t.dtype);
            p = put<uint8_t>(p, (uint8_t)t.ndim);
            p = put<uint8_t>(p, 0);
            p = put<uint8_t>(p, 0);
            for (int k = 0; k < t.ndim; ++k) p = put<uint32_t>(p, t.dims[k]);
            p = put<float>(p, t.scale);
            p = put<uint32_t>(p, 0u);           // tensor flags
            p = put<uint64_t>(p, L.offsets[i]);
            p = put<uint64_t>(p, t.byte_len);
        }
        std::memset(p, 0, (size_t)(out + L.payload_start - p));  // up to the payload start
        uint8_t *payload = out + L.payload_start;
        std::memset(payload, 0, (size_t)L.payload_len);
        for (int64_t i = 0; i < n; ++i)
            if (tensors[i].byte_len) std::memcpy(payload + L.offsets[(size_t)i], tensors[i].data, (size_t)tensors[i].byte_len);
        if (with_hash) put<uint64_t>(hash_at, bpw_fnv1a64(payload, (size_t)L.payload_len));
        *written = total;
    } catch (const std::bad_alloc &) {
        return tfail(err, BPW_E_INVAL, 0, -1, -1, "out of host memory");
    }
    return BPW_OK;
}

}  // extern "C"

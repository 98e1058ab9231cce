// Host-only driver for libbpw's untrusted-input paths, built with AddressSanitizer and
// UndefinedBehaviorSanitizer from the library's own host sources (container reader, plane
// packer / validator / loader, BITCOS packers). The GPU launchers and the few HIP runtime calls
// those sources reference are replaced below by stubs that abort if reached: no case here
// launches work, so reaching one is itself a failure.
//
// Input (argv[1]): a sequence of little-endian records
//     u32 op, u32 flags, i64 rows, i64 cols, u64 len, u8 data[len]
// Each record's bytes are copied into a buffer of exactly `len` bytes (NULL when len is 0), so
// a read one byte past the end is an ASan report. Output: one line per record on stdout.
//   op 1, container: open, then verify when flags & 1 (hash when flags & 2):
//       "<check> <tensor> <row> <beat> <col>" and, when it opened,
//       " | <count> <stored hash> <config bytes>" and per tensor " <dtype>:<find>:<load status>:<row>:<beat>:<col>"
//   op 2, planes: bpw_validate, then bpw_load with scale 1:
//       "<status> <row> <beat> <col> <load status>"
//   op 3, int8 trits [rows x cols]: bpw_pack_i8, bpw_bitcos_pack_i8 and, when packing succeeded,
//       bpw_load + bpw_bitcos_from_planes:
//       "<status> <row> <beat> <col> <planes fnv>" " / <status> <row> <beat> <col> <bitcos>" [" / <bitcos>"]
//       with <bitcos> = "<presence fnv> <signs fnv> <row_start fnv> <nnz> <sign words> <device bytes>".
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/bpw.h"
#include "../../bit_plane_weight_amd/csrc/bpw_internal.h"

// ------------------------------------------------------------------ stubs (never reached)

[[noreturn]] static void unreachable(const char *what) {
    std::fprintf(stderr, "host driver: %s reached\n", what);
    std::abort();
}

extern "C" {
hipError_t hipGetDevice(int *) { unreachable("hipGetDevice"); }
hipError_t hipDeviceGetAttribute(int *, hipDeviceAttribute_t, int) { unreachable("hipDeviceGetAttribute"); }
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *, int) { unreachable("hipGetDeviceProperties"); }
const char *hipGetErrorString(hipError_t) { unreachable("hipGetErrorString"); }
hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t) {
    unreachable("hipMemcpyAsync");
}
hipError_t hipStreamSynchronize(hipStream_t) { unreachable("hipStreamSynchronize"); }
}

namespace bpw {
int launch_gemv_bytelane(const DevJob *, const Tile *, int32_t, void *) { unreachable("a launcher"); }
int launch_gemv_bitserial(const DevJob *, const Tile *, int32_t, void *) { unreachable("a launcher"); }
int launch_gemm_small_batch(const SmallBatchArgs &, int32_t, int32_t, void *) { unreachable("a launcher"); }
int launch_gemm_small_batch_mfma(const SmallBatchArgs &, void *) { unreachable("a launcher"); }
int launch_gemm_small_batch_grouped(const SmallBatchArgs *, const SBTile *, int32_t, void *) {
    unreachable("a launcher");
}
int launch_gemv_tokens(const TokJob *, const Tile *, int32_t, int32_t, void *) { unreachable("a launcher"); }
int launch_gemv_bitcos(const BitcosJob *, const Tile *, int32_t, void *) { unreachable("a launcher"); }
int launch_dense_head(const uint16_t *, int64_t, int64_t, const uint16_t *, float *, void *) {
    unreachable("a launcher");
}
int launch_quantize(const QuantJob *, int32_t, void *) { unreachable("a launcher"); }
int launch_probe(const void *, size_t, uint32_t *, int32_t, void *) { unreachable("a launcher"); }
int launch_flush(void *, size_t, void *) { unreachable("a launcher"); }
int static_scratch(void **, size_t *) { unreachable("static_scratch"); }
}  // namespace bpw

// ------------------------------------------------------------------ cases

namespace {

struct Buf {  // exactly len bytes on the heap, NULL when empty
    uint8_t *p = nullptr;
    size_t n = 0;
    explicit Buf(size_t len) : n(len) {
        if (len) {
            p = static_cast<uint8_t *>(std::malloc(len));
            if (!p) unreachable("out of memory");
        }
    }
    ~Buf() { std::free(p); }
    Buf(const Buf &) = delete;
    Buf &operator=(const Buf &) = delete;
};

std::string fmt(const char *f, ...) __attribute__((format(printf, 1, 2)));
std::string fmt(const char *f, ...) {
    char b[512];
    va_list ap;
    va_start(ap, f);
    std::vsnprintf(b, sizeof b, f, ap);
    va_end(ap);
    return b;
}

uint64_t fnv_of(const void *p, size_t n) { return bpw_fnv1a64(static_cast<const uint8_t *>(p), n); }

std::string container_case(const Buf &b, uint32_t flags) {
    bpw_trit_file *f = nullptr;
    bpw_trit_err e;
    std::memset(&e, 0, sizeof e);
    std::string out;
    bpw_status st = bpw_trit_open(b.p, b.n, &f, &e);
    if (st == BPW_OK && (flags & 1)) st = bpw_trit_verify(f, (flags & 2) ? 1 : 0, &e);
    if (st != BPW_OK)
        out = fmt("%d %lld %lld %lld %lld", e.check, (long long)e.tensor, (long long)e.row, (long long)e.beat,
                  (long long)e.col);
    else
        out = "0 -1 -1 -1 -1";
    if (!f) return out;
    const char *json = nullptr;
    size_t json_len = 0;
    if (bpw_trit_config(f, &json, &json_len) != BPW_OK) unreachable("bpw_trit_config failed on an open file");
    const int64_t n = bpw_trit_tensor_count(f);
    out += fmt(" | %lld %llu %zu", (long long)n, (unsigned long long)bpw_trit_stored_hash(f), json_len);
    for (int64_t i = 0; i < n; ++i) {
        bpw_trit_tensor t;
        if (bpw_trit_tensor_info(f, i, &t) != BPW_OK) unreachable("bpw_trit_tensor_info failed in range");
        // touch every byte the record claims, so a wrong pointer or length is an ASan report
        volatile uint64_t h = fnv_of(t.data, t.byte_len) ^ fnv_of(t.name, (size_t)t.name_len);
        (void)h;
        const int64_t found = bpw_trit_find(f, t.name, (size_t)t.name_len);
        bpw_host_mat *m = nullptr;
        bpw_err le = {BPW_OK, -1, -1, -1};
        const bpw_status ls = bpw_trit_load(f, i, &m, &le);
        if (ls == BPW_OK && bpw_host_mat_bytes(m) != t.byte_len) unreachable("loaded size differs");
        bpw_host_mat_free(m);
        out += fmt(" %d:%lld:%d:%lld:%lld:%lld", t.dtype, (long long)found, (int)ls,
                   ls == BPW_OK ? -1LL : (long long)le.row, ls == BPW_OK ? -1LL : (long long)le.beat,
                   ls == BPW_OK ? -1LL : (long long)le.col);
    }
    if (bpw_trit_tensor_info(f, n, nullptr) == BPW_OK) unreachable("tensor_info accepted an index past the end");
    bpw_trit_close(f);
    return out;
}

std::string planes_case(const Buf &b, int64_t rows, int64_t cols) {
    bpw_err e = {BPW_OK, -1, -1, -1};
    const bpw_status st = bpw_validate(b.p, b.n, rows, cols, &e);
    bpw_host_mat *m = nullptr;
    bpw_err le = {BPW_OK, -1, -1, -1};
    const bpw_status ls = bpw_load(b.p, b.n, rows, cols, 1.0f, &m, &le);
    if (ls == BPW_OK && bpw_host_mat_bytes(m) != b.n) unreachable("loaded size differs");
    bpw_host_mat_free(m);
    if (st == BPW_OK) return fmt("0 -1 -1 -1 %d", (int)ls);
    return fmt("%d %lld %lld %lld %d", (int)st, (long long)e.row, (long long)e.beat, (long long)e.col, (int)ls);
}

std::string bitcos_summary(const bpw_bitcos_host *h, int64_t rows, int64_t cols) {
    const uint64_t *p = nullptr;
    const uint32_t *s = nullptr, *r = nullptr;
    int64_t sw = 0, nnz = 0;
    if (bpw_bitcos_arrays(h, &p, &s, &r, &sw, &nnz) != BPW_OK) unreachable("bpw_bitcos_arrays failed");
    const size_t bpr = (size_t)((cols + 63) / 64);
    return fmt("%llu %llu %llu %lld %lld %zu", (unsigned long long)fnv_of(p, (size_t)rows * bpr * 8),
               (unsigned long long)fnv_of(s, (size_t)sw * 4), (unsigned long long)fnv_of(r, (size_t)(rows + 1) * 4),
               (long long)nnz, (long long)sw, bpw_bitcos_device_bytes(h));
}

std::string trits_case(const Buf &b, int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0 || (uint64_t)rows * (uint64_t)cols != b.n) unreachable("trit record size");
    const size_t bpr = (size_t)((cols + 63) / 64);
    Buf planes((size_t)rows * bpr * 16);
    bpw_err e = {BPW_OK, -1, -1, -1};
    const bpw_status st = bpw_pack_i8(reinterpret_cast<const int8_t *>(b.p), rows, cols, planes.p, planes.n, &e);
    std::string out = st == BPW_OK ? fmt("0 -1 -1 -1 %llu", (unsigned long long)fnv_of(planes.p, planes.n))
                                   : fmt("%d %lld %lld %lld 0", (int)st, (long long)e.row, (long long)e.beat,
                                         (long long)e.col);
    bpw_bitcos_host *h = nullptr;
    bpw_err be = {BPW_OK, -1, -1, -1};
    const bpw_status bs = bpw_bitcos_pack_i8(reinterpret_cast<const int8_t *>(b.p), rows, cols, 0.5f, &h, &be);
    if (bs == BPW_OK)
        out += " / 0 -1 -1 -1 " + bitcos_summary(h, rows, cols);
    else
        out += fmt(" / %d %lld %lld %lld", (int)bs, (long long)be.row, (long long)be.beat, (long long)be.col);
    bpw_bitcos_free(h);
    if (st == BPW_OK) {
        bpw_host_mat *m = nullptr;
        bpw_err le = {BPW_OK, -1, -1, -1};
        if (bpw_load(planes.p, planes.n, rows, cols, 0.5f, &m, &le) != BPW_OK) unreachable("packed planes refused");
        bpw_bitcos_host *g = nullptr;
        const bpw_status gs = bpw_bitcos_from_planes(m, &g);
        out += gs == BPW_OK ? " / " + bitcos_summary(g, rows, cols) : fmt(" / %d", (int)gs);
        bpw_bitcos_free(g);
        bpw_host_mat_free(m);
    }
    return out;
}

// Open a container and write its tensors and config again with bpw_trit_write (flags bit 0: store the
// payload hash). The output is the write's check and location, or its size and FNV-1a-64; a file the
// writer accepted must reopen and verify.
std::string rewrite_case(const Buf &b, uint32_t flags) {
    bpw_trit_file *f = nullptr;
    bpw_trit_err e;
    std::memset(&e, 0, sizeof e);
    if (bpw_trit_open(b.p, b.n, &f, &e) != BPW_OK)
        return fmt("open %d %lld", e.check, (long long)e.tensor);
    const char *json = nullptr;
    size_t json_len = 0;
    if (bpw_trit_config(f, &json, &json_len) != BPW_OK) unreachable("bpw_trit_config failed on an open file");
    const int64_t n = bpw_trit_tensor_count(f);
    std::vector<bpw_trit_tensor_in> in((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        bpw_trit_tensor t;
        if (bpw_trit_tensor_info(f, i, &t) != BPW_OK) unreachable("bpw_trit_tensor_info failed in range");
        bpw_trit_tensor_in &w = in[(size_t)i];
        w.name = t.name;
        w.name_len = t.name_len;
        w.dtype = t.dtype;
        w.ndim = t.ndim;
        for (int k = 0; k < 4; ++k) w.dims[k] = t.dims[k];
        w.scale = t.scale;
        w.reserved = 0;
        w.data = t.data;
        w.byte_len = t.byte_len;
    }
    uint64_t need = 0;
    if (bpw_trit_write_size(in.data(), n, json_len, &need, &e) != BPW_OK) unreachable("an opened file's tensors refused");
    Buf out((size_t)need);
    uint64_t written = 0;
    const bpw_status st = bpw_trit_write(in.data(), n, json, json_len, (int32_t)(flags & 1), out.p, out.n, &written, &e);
    std::string line;
    if (st != BPW_OK) {
        line = fmt("%d %lld %lld %lld %lld", e.check, (long long)e.tensor, (long long)e.row, (long long)e.beat,
                   (long long)e.col);
    } else {
        if (written != need) unreachable("written size differs from the computed one");
        bpw_trit_file *g = nullptr;
        if (bpw_trit_open(out.p, out.n, &g, &e) != BPW_OK || bpw_trit_verify(g, 1, &e) != BPW_OK)
            unreachable("a written container does not open and verify");
        bpw_trit_close(g);
        line = fmt("0 | %llu %llu", (unsigned long long)written, (unsigned long long)fnv_of(out.p, out.n));
    }
    bpw_trit_close(f);
    return line;
}

}  // namespace

int main(int argc, char **argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s <cases>\n", argv[0]);
        return 2;
    }
    FILE *in = std::fopen(argv[1], "rb");
    if (!in) {
        std::perror(argv[1]);
        return 2;
    }
    long cases = 0;
    for (;;) {
        struct {
            uint32_t op, flags;
            int64_t rows, cols;
            uint64_t len;
        } hd;
        const size_t got = std::fread(&hd, 1, sizeof hd, in);
        if (got == 0 && std::feof(in)) break;
        if (got != sizeof hd || hd.len > (1ull << 32)) unreachable("a malformed case file");
        Buf b((size_t)hd.len);
        if (hd.len && std::fread(b.p, 1, b.n, in) != b.n) unreachable("a short case file");
        std::string line;
        switch (hd.op) {
            case 1: line = container_case(b, hd.flags); break;
            case 2: line = planes_case(b, hd.rows, hd.cols); break;
            case 3: line = trits_case(b, hd.rows, hd.cols); break;
            case 4: line = rewrite_case(b, hd.flags); break;
            default: unreachable("an unknown case op");
        }
        std::fputs(line.c_str(), stdout);
        std::fputc('\n', stdout);
        ++cases;
    }
    std::fclose(in);
    std::fprintf(stderr, "host driver: %ld cases\n", cases);
    return 0;
}

// bpw_measure.hip - measurement helpers: streaming-read probe and cache flush.
//
// Written for CDNA4 (wave64); launched only by bpw_host.cpp after its argument and architecture
// checks.
#include "bpw_device.h"

namespace bpw {

// Measurement helpers.

// Streaming-read probe: plain reads of a buffer in the pattern the dense head streams with. Each
// workgroup of T threads reads one contiguous chunk of L * T * 16 bytes, every lane issuing all of its
// L non-temporal 16-byte loads before it uses the first (one wave covers L KiB, 1 KiB per load
// instruction), and workgroups are renumbered so that each XCD (workgroup b runs on XCD b mod xcds)
// streams one contiguous run of chunks. Shapes differ in L, T and the load kind (buffer loads, where
// bytes past the end read zeros through the range check, or global loads guarded per lane); the probe
// of a measurement is the best of them. A data-dependent store keeps every load alive.
template <int L, int T, bool BUF>
__global__ __launch_bounds__(T) void stream_probe_kernel(const uint8_t *__restrict__ p, int64_t len,
                                                         uint32_t *__restrict__ sink, int xcds) {
    constexpr int64_t kChunk = (int64_t)L * T * 16;
    const int64_t nb = gridDim.x, b = blockIdx.x, xc = b % xcds, per = nb / xcds, extra = nb % xcds;
    const int64_t chunk = xc * per + (xc < extra ? xc : extra) + b / xcds;
    const int64_t base = chunk * kChunk;
    const int64_t left = len - base;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t off0 = (uint32_t)(wave * L * 1024 + lane * 16);
    u32x4 v[L];
    if constexpr (BUF) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(p + base, (uint32_t)(left < kChunk ? left : kChunk));
#pragma unroll
        for (int k = 0; k < L; ++k) v[k] = load_beat(r, off0 + 1024u * k);
    } else {
#pragma unroll
        for (int k = 0; k < L; ++k) {
            const int64_t o = (int64_t)off0 + 1024 * k;
            v[k] = o + 16 <= left ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + base + o))
                                  : u32x4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < L; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    if (acc == 0x9E3779B9u) sink[0] = acc;  // data-dependent store keeps every load alive
}

__global__ __launch_bounds__(kThreads) void flush_kernel(u32x4 *__restrict__ p, int64_t n, uint32_t key) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        u32x4 v = p[i];
        v.x ^= key;
        p[i] = v;
    }
}

// ------------------------------------------------------------------------------------------
// Launchers.

template <int L, int T, bool BUF>
static int probe_launch(const void *buf, size_t len, uint32_t *sink, void *stream) {
    constexpr int64_t kChunk = (int64_t)L * T * 16;
    const int64_t chunks = ((int64_t)len + kChunk - 1) / kChunk;
    hipLaunchKernelGGL((stream_probe_kernel<L, T, BUF>), dim3((unsigned)chunks), dim3(T), 0, as_stream(stream),
                       reinterpret_cast<const uint8_t *>(buf), (int64_t)len, sink, host_xcds());
    return hipGetLastError();
}

int launch_probe(const void *buf, size_t len, uint32_t *sink, int32_t shape, void *stream) {
    if (len == 0) return hipSuccess;
    switch (shape) {
        case 0: return probe_launch<10, 256, true>(buf, len, sink, stream);
        case 1: return probe_launch<10, 256, false>(buf, len, sink, stream);
        case 2: return probe_launch<8, 512, true>(buf, len, sink, stream);
        case 3: return probe_launch<8, 512, false>(buf, len, sink, stream);
        case 4: return probe_launch<4, 256, true>(buf, len, sink, stream);
        default: return hipErrorInvalidValue;
    }
}

int launch_flush(void *buf, size_t len, void *stream) {
    const int64_t n = (int64_t)(len / 16);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(flush_kernel, dim3(256 * 16), dim3(kThreads), 0, as_stream(stream),
                       reinterpret_cast<u32x4 *>(buf), n, 0u);
    return hipGetLastError();
}

}  // namespace bpw

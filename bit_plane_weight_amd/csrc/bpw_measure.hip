// bpw_measure.hip - measurement helpers: streaming-read probe and cache flush.
//
// Written for CDNA4 (wave64); launched only by bpw_host.cpp after its argument and architecture
// checks.
#include "bpw_device.h"

namespace bpw {

// Measurement helpers.

// Streaming-read probe, the best plain read pattern measured on this part (the one the dense head
// streams with): each workgroup of kThreads reads one contiguous chunk of kProbeLoads * 4 KiB, every
// lane issuing all of its kProbeLoads non-temporal 16-byte loads before it uses the first (one wave
// covers kProbeLoads KiB, 1 KiB per load instruction), and workgroups are renumbered so that each XCD
// (workgroup b runs on XCD b mod xcds) streams one contiguous run of chunks. Bytes past the end of the
// buffer read zeros through the buffer range check. A data-dependent store keeps every load alive.
constexpr int kProbeLoads = 10;
constexpr int64_t kProbeChunk = (int64_t)kProbeLoads * kThreads * 16;

__global__ __launch_bounds__(kThreads) void stream_probe_kernel(const uint8_t *__restrict__ p, int64_t len,
                                                                uint32_t *__restrict__ sink, int xcds) {
    const int64_t nb = gridDim.x, b = blockIdx.x, xc = b % xcds, per = nb / xcds, extra = nb % xcds;
    const int64_t chunk = xc * per + (xc < extra ? xc : extra) + b / xcds;
    const int64_t base = chunk * kProbeChunk;
    const int64_t left = len - base;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(p + base, (uint32_t)(left < kProbeChunk ? left : kProbeChunk));
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t off0 = (uint32_t)(wave * kProbeLoads * 1024 + lane * 16);
    u32x4 v[kProbeLoads];
#pragma unroll
    for (int k = 0; k < kProbeLoads; ++k) v[k] = load_beat(r, off0 + 1024u * k);
    uint32_t acc = 0;
#pragma unroll
    for (int k = 0; k < kProbeLoads; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
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

int launch_probe(const void *buf, size_t len, uint32_t *sink, void *stream) {
    if (len == 0) return hipSuccess;
    const int64_t chunks = ((int64_t)len + kProbeChunk - 1) / kProbeChunk;
    hipLaunchKernelGGL(stream_probe_kernel, dim3((unsigned)chunks), dim3(kThreads), 0, as_stream(stream),
                       reinterpret_cast<const uint8_t *>(buf), (int64_t)len, sink, host_xcds());
    return hipGetLastError();
}

int launch_flush(void *buf, size_t len, void *stream) {
    const int64_t n = (int64_t)(len / 16);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(flush_kernel, dim3(256 * 16), dim3(kThreads), 0, as_stream(stream),
                       reinterpret_cast<u32x4 *>(buf), n, 0u);
    return hipGetLastError();
}

}  // namespace bpw

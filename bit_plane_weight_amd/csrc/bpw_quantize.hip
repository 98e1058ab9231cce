// bpw_quantize.hip - Folded activation quantiser on gfx950 ("Tritium: One Weight Format for Ternary
// Inference on Commodity CPUs and Multiplier-Free Hardware", "Numerics": absmax codes are invariant
// under a uniform positive scale, so they are taken from h * g and the RMS norm's 1/rms survives only
// in the per-token scale; no per-element divide by rms).
//
// One workgroup per activation: pass 1 forms u = h * g (float32) for its max |u| and sums h^2 in
// float64; pass 2 writes q = rint((127 * u) / m) as int8 (float32 multiply, correctly rounded divide,
// ties to even) and zeros up to q_len; thread 0 writes scale = (float)((m / 127) / sqrt(ss / n + eps))
// in float64. The codes use the same float32 operations in the same order for every element, so they
// do not depend on the launch shape; the float64 sum of squares does (in its last bits only).
#include "bpw_device.h"

namespace bpw {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__global__ __launch_bounds__(kThreads) void quantize_kernel(const QuantJob *__restrict__ jobs) {
    __shared__ float smax[kWaves];
    __shared__ double ssum[kWaves];
    const QuantJob J = jobs[blockIdx.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float m = 0.0f;
    double ss = 0.0;
    for (int64_t i = threadIdx.x; i < J.n; i += kThreads) {
        const float h = J.h[i];
        const float u = h * J.g[i];
        m = fmaxf(m, fabsf(u));
        ss += (double)h * (double)h;  // exact product of two floats
    }
    m = wave_max(m);
    ss = wave_sum(ss);
    if (lane == 0) {
        smax[wave] = m;
        ssum[wave] = ss;
    }
    __syncthreads();
    m = smax[0];
    ss = ssum[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        m = fmaxf(m, smax[w]);
        ss += ssum[w];
    }
    for (int64_t i = threadIdx.x; i < J.q_len; i += kThreads) {
        int8_t code = 0;
        if (i < J.n && m > 0.0f) {
            const float u = J.h[i] * J.g[i];
            float r = rintf((127.0f * u) / m);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            code = (int8_t)r;
        }
        J.q[i] = code;
    }
    if (threadIdx.x == 0) {
        const double rms = sqrt(ss / (double)J.n + (double)J.eps);
        *J.scale = m > 0.0f ? (float)(((double)m / 127.0) / rms) : 0.0f;
    }
}

int launch_quantize(const QuantJob *jobs, int32_t n_jobs, void *stream) {
    if (n_jobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)n_jobs), dim3(kThreads), 0, as_stream(stream), jobs);
    return hipGetLastError();
}

}  // namespace bpw

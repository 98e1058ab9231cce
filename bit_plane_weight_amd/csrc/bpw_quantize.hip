// bpw_quantize.hip - Folded activation quantiser on gfx950 ("Tritium: One Weight Format for Ternary
// Inference on Commodity CPUs and Multiplier-Free Hardware", "Numerics": absmax codes are invariant
// under a uniform positive scale, so they are taken from h * g and the RMS norm's 1/rms survives only
// in the per-token scale; no per-element divide by rms).
//
// One workgroup per activation: it forms u = h * g (float32), its max |u| and the float64 sum of
// h^2, then writes q = rint((127 * u) / m) as int8 (float32 multiply, correctly rounded divide, ties
// to even) and zeros up to q_len; thread 0 writes scale = (float)((m / 127) / sqrt(ss / n + eps)) in
// float64. The codes use the same float32 operations in the same order for every element, so they
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

// Max |u| and sum h^2 over the workgroup (all threads get both).
__device__ __forceinline__ void block_reduce(float &m, double &ss, float *smax, double *ssum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
}

// One code. A code whose float32 value is NaN (a NaN input, or an infinite one once m is infinite)
// is 0; NaN inputs never raise m (fmaxf drops a NaN operand). Finite values clamp to +-127.
__device__ __forceinline__ int8_t code_of(float u, float m) {
    if (!(m > 0.0f)) return 0;
    const float r = rintf((127.0f * u) / m);
    if (r != r) return 0;
    return (int8_t)fminf(fmaxf(r, -127.0f), 127.0f);
}

__device__ __forceinline__ void write_scale(const QuantJob &J, float m, double ss) {
    if (threadIdx.x == 0) {
        const double rms = sqrt(ss / (double)J.n + (double)J.eps);
        *J.scale = m > 0.0f ? (float)(((double)m / 127.0) / rms) : 0.0f;
    }
}

// Vectors of up to kQuantHeld * kThreads elements: each thread keeps its u values in registers, so
// every load is issued before the first is used and h, g are read once.
constexpr int kQuantHeld = 32;

__global__ __launch_bounds__(kThreads) void quantize_kernel(const QuantJob *__restrict__ jobs) {
    __shared__ float smax[kWaves];
    __shared__ double ssum[kWaves];
    const QuantJob J = jobs[blockIdx.x];
    float m = 0.0f;
    double ss = 0.0;
    if (J.n <= (int64_t)kQuantHeld * kThreads) {
        float u[kQuantHeld];
#pragma unroll
        for (int k = 0; k < kQuantHeld; ++k) {
            const int64_t i = threadIdx.x + (int64_t)k * kThreads;
            const float h = i < J.n ? J.h[i] : 0.0f;
            const float g = i < J.n ? J.g[i] : 0.0f;
            u[k] = h * g;
            m = fmaxf(m, fabsf(u[k]));
            ss += (double)h * (double)h;  // exact product of two floats
        }
        block_reduce(m, ss, smax, ssum);
#pragma unroll
        for (int k = 0; k < kQuantHeld; ++k) {
            const int64_t i = threadIdx.x + (int64_t)k * kThreads;
            if (i < J.q_len) J.q[i] = i < J.n ? code_of(u[k], m) : (int8_t)0;
        }
        for (int64_t i = threadIdx.x + (int64_t)kQuantHeld * kThreads; i < J.q_len; i += kThreads) J.q[i] = 0;
    } else {  // longer vectors: two passes over h and g
        for (int64_t i = threadIdx.x; i < J.n; i += kThreads) {
            const float h = J.h[i];
            m = fmaxf(m, fabsf(h * J.g[i]));
            ss += (double)h * (double)h;
        }
        block_reduce(m, ss, smax, ssum);
        for (int64_t i = threadIdx.x; i < J.q_len; i += kThreads) J.q[i] = i < J.n ? code_of(J.h[i] * J.g[i], m) : (int8_t)0;
    }
    write_scale(J, m, ss);
}

int launch_quantize(const QuantJob *jobs, int32_t n_jobs, void *stream) {
    if (n_jobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)n_jobs), dim3(kThreads), 0, as_stream(stream), jobs);
    return hipGetLastError();
}

}  // namespace bpw

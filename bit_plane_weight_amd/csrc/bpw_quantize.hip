// bpw_quantize.hip - Folded activation quantiser on gfx950 ("Tritium: One Weight Format for Ternary
// Inference on Commodity CPUs and Multiplier-Free Hardware", "Numerics": absmax codes are invariant
// under a uniform positive scale, so they are taken from h * g and the RMS norm's 1/rms survives only
// in the per-token scale; no per-element divide by rms).
//
// One workgroup of 16 waves per activation: it forms u = h * g (float32), its max |u| and the float64
// sum of h^2, writes scale = (float)((m / 127) / sqrt(ss / n + eps)) in float64 (one lane of the last
// wave), then q = rint((127 * u) / m) as int8 (float32 multiply, correctly rounded divide, ties to
// even) and zeros up to q_len. The codes use the same float32 operations in the same order for every element, so they
// do not depend on the launch shape; the float64 sum of squares does (in its last bits only).
#include "bpw_device.h"

namespace bpw {

// Workgroup shape: 16 waves, so a 6912-element activation is 7 elements per thread.
constexpr int kQWaves = 16;
constexpr int kQThreads = 64 * kQWaves;

// Row-of-16 steps by DPP (swap pairs, swap halves of a quad, mirror within 8, mirror within 16): after
// them every lane of a row holds its row's result; the four rows are then combined from lanes 0, 16,
// 32 and 48 read as scalars. DPP moves cost a few cycles where a cross-lane shuffle through LDS
// (ds_bpermute) costs an LDS round trip per step.
__device__ __forceinline__ float dpp_f(float v, int ctrl_sel) {
    const int x = __builtin_bit_cast(int, v);
    int r;
    switch (ctrl_sel) {
        case 0: r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;
        case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;
        default: r = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break;
    }
    return __builtin_bit_cast(float, r);
}

__device__ __forceinline__ double dpp_d(double v, int ctrl_sel) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
    int rl, rh;
    switch (ctrl_sel) {
        case 0:
            rl = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, false);
            rh = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, false);
            break;
        case 1:
            rl = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, false);
            rh = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, false);
            break;
        case 2:
            rl = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, false);
            rh = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, false);
            break;
        default:
            rl = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xF, 0xF, false);
            rh = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xF, 0xF, false);
            break;
    }
    return __builtin_bit_cast(double, ((uint64_t)(uint32_t)rh << 32) | (uint32_t)rl);
}

__device__ __forceinline__ float lane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

__device__ __forceinline__ double lane_d(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Max over the wave (every lane gets it). fmaxf drops a NaN operand, in any order.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v = fmaxf(v, dpp_f(v, c));
    return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Sum over the wave (every lane gets it); the order is fixed by the lane layout.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int c = 0; c < 4; ++c) v += dpp_d(v, c);
    return (lane_d(v, 0) + lane_d(v, 16)) + (lane_d(v, 32) + lane_d(v, 48));
}

// The last wave holds the fewest codes for the decode step's widths (2560, 6912), so it finishes the
// sum of h^2 and writes the scale while the others are still writing codes.
constexpr int kScaleWave = kQWaves - 1;

// Max |u| over the workgroup for every thread; the sum of h^2 for the scale's wave only.
// The sixteen per-wave values are combined as a balanced tree.
__device__ __forceinline__ void block_reduce(float &m, double &ss, float *smax, double *ssum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    m = wave_max(m);
    ss = wave_sum(ss);
    if (lane == 0) {
        smax[wave] = m;
        ssum[wave] = ss;
    }
    __syncthreads();
    float w[kQWaves];
#pragma unroll
    for (int i = 0; i < kQWaves; ++i) w[i] = smax[i];
#pragma unroll
    for (int h = kQWaves / 2; h >= 1; h /= 2)
#pragma unroll
        for (int i = 0; i < h; ++i) w[i] = fmaxf(w[i], w[i + h]);
    m = w[0];
    if (wave == kScaleWave) {
        double d[kQWaves];
#pragma unroll
        for (int i = 0; i < kQWaves; ++i) d[i] = ssum[i];
#pragma unroll
        for (int h = kQWaves / 2; h >= 1; h /= 2)
#pragma unroll
            for (int i = 0; i < h; ++i) d[i] += d[i + h];
        ss = d[0];
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

// The scale, written by lane 0 of the scale's wave right after the reductions (before the codes).
__device__ __forceinline__ void write_scale(const QuantJob &J, float m, double ss) {
    if (threadIdx.x == kScaleWave * 64) {
        const double rms = sqrt(ss / (double)J.n + (double)J.eps);
        *J.scale = m > 0.0f ? (float)(((double)m / 127.0) / rms) : 0.0f;
    }
}

// Vectors of up to kQuantHeld * kQThreads elements: each thread keeps its u values in registers, so
// every load is issued before the first is used and h, g are read once.
constexpr int kQuantHeld = 8;

__global__ __launch_bounds__(kQThreads) void quantize_kernel(const QuantJob *__restrict__ jobs) {
    __shared__ float smax[kQWaves];
    __shared__ double ssum[kQWaves];
    const QuantJob J = jobs[blockIdx.x];
    float m = 0.0f;
    double ss = 0.0;
    if (J.n <= (int64_t)kQuantHeld * kQThreads) {
        float u[kQuantHeld];
#pragma unroll
        for (int k = 0; k < kQuantHeld; ++k) {
            const int64_t i = threadIdx.x + (int64_t)k * kQThreads;
            const float h = i < J.n ? J.h[i] : 0.0f;
            const float g = i < J.n ? J.g[i] : 0.0f;
            u[k] = h * g;
            m = fmaxf(m, fabsf(u[k]));
            ss += (double)h * (double)h;  // exact product of two floats
        }
        block_reduce(m, ss, smax, ssum);
        write_scale(J, m, ss);
#pragma unroll
        for (int k = 0; k < kQuantHeld; ++k) {
            const int64_t i = threadIdx.x + (int64_t)k * kQThreads;
            if (i < J.q_len) J.q[i] = i < J.n ? code_of(u[k], m) : (int8_t)0;
        }
        for (int64_t i = threadIdx.x + (int64_t)kQuantHeld * kQThreads; i < J.q_len; i += kQThreads) J.q[i] = 0;
    } else {  // longer vectors: two passes over h and g
        for (int64_t i = threadIdx.x; i < J.n; i += kQThreads) {
            const float h = J.h[i];
            m = fmaxf(m, fabsf(h * J.g[i]));
            ss += (double)h * (double)h;
        }
        block_reduce(m, ss, smax, ssum);
        write_scale(J, m, ss);
        for (int64_t i = threadIdx.x; i < J.q_len; i += kQThreads) J.q[i] = i < J.n ? code_of(J.h[i] * J.g[i], m) : (int8_t)0;
    }
}

int launch_quantize(const QuantJob *jobs, int32_t n_jobs, void *stream) {
    if (n_jobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)n_jobs), dim3(kQThreads), 0, as_stream(stream), jobs);
    return hipGetLastError();
}

}  // namespace bpw

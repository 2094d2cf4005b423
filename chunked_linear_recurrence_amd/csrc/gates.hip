// Gate transform for gfx950: raw gate projections to the float32 natural-log decays the chunk
// and recurrent paths consume (attention-gym "Linear Attention", section "Gate Transforms").
// Element e of raw [rows, H, D] (D = 1 for per-head gates), with j = e mod (H D), h = j / D:
//   softplus kind:  g = -exp(A_log[h]) * softplus(raw[e] + dt_bias[j])
//   bounded kind:   g = lower_bound * sigmoid(exp(A_log[h]) * (raw[e] + dt_bias[j]))
// An elementwise pass bound by HBM: each thread moves four consecutive elements per step
// (8 or 16 bytes in, 16 bytes out) over a grid-stride loop sized to fill the GPU, with the
// exponential and logarithm of the hardware (v_exp_f32, v_log_f32).
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {
namespace {

template <typename ET> struct In4;
template <> struct In4<float> {
    static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ float load1(const float* p) { return *p; }
};
template <> struct In4<bf16_t> {
    static __device__ __forceinline__ f32x4 load(const bf16_t* p) {
        return Elem<bf16_t>::unpack(*reinterpret_cast<const i16x4*>(p));
    }
    static __device__ __forceinline__ float load1(const bf16_t* p) { return bf2f(*p); }
};

constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;

// a = raw + bias; amp2 = exp(A_log) log2(e)
template <bool BOUNDED>
__device__ __forceinline__ float transform(float a, float amp2, float lb) {
    if constexpr (BOUNDED) {
        // lower_bound * sigmoid(exp(A_log) a) = lower_bound / (1 + 2^(-amp2 a))
        return lb * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-amp2 * a));
    } else {
        // -exp(A_log) softplus(a), softplus(a) = max(a, 0) + ln 2 log2(1 + 2^(-|a| log2 e)) (never overflows)
        const float sp = fmaxf(a, 0.f) + kLn2 * __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(a) * kLog2e));
        return -(amp2 * kLn2) * sp;
    }
}

// The launch makes 4 * (threads in the grid) a multiple of H*D, so every thread meets the same
// four channel positions j0..j0+3 (mod H*D) on each sweep and reads their parameters once.
template <typename ET, bool BOUNDED>
__global__ __launch_bounds__(256) void gate_transform_kernel(const ET* __restrict__ raw, const float* __restrict__ A_log,
                                                             const float* __restrict__ dt_bias, long n, int H, int D,
                                                             float lb, float* __restrict__ out) {
    const int HD = H * D;
    const long n4 = n / 4, stride = (long)gridDim.x * blockDim.x;
    const long i0 = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int j0 = (int)((4 * i0) % HD);
    float bias[4], amp2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = (j0 + e) % HD;
        bias[e] = dt_bias[j];
        amp2[e] = expf(A_log[j / D]) * kLog2e;
    }
    for (long i = i0; i < n4; i += stride) {
        const f32x4 x = In4<ET>::load(raw + 4 * i);
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = transform<BOUNDED>(x[e] + bias[e], amp2[e], lb);
        *reinterpret_cast<f32x4*>(out + 4 * i) = y;
    }
    // the last n mod 4 elements
    if (blockIdx.x == 0 && threadIdx.x < n - 4 * n4) {
        const long e = 4 * n4 + threadIdx.x;
        const int j = (int)(e % HD);
        out[e] = transform<BOUNDED>(In4<ET>::load1(raw + e) + dt_bias[j], expf(A_log[j / D]) * kLog2e, lb);
    }
}

template <typename ET>
hipError_t launch_typed(bool bounded, const void* raw, const float* A_log, const float* dt_bias, long n, int H, int D,
                        float lb, float* out, hipStream_t s) {
    // enough blocks to fill the GPU, rounded up to a multiple of H*D / gcd(H*D, 1024) (one sweep of
    // the grid moves 1024 elements per block)
    const long HD = (long)H * D;
    long a = HD, bb = 1024;
    while (bb) {
        const long t = a % bb;
        a = bb;
        bb = t;
    }
    const long m = HD / a;
    long want = (n / 4 + 255) / 256;
    if (want > 4096) want = 4096;
    if (want < 1) want = 1;
    const unsigned grid = (unsigned)(((want + m - 1) / m) * m);
    const ET* r = static_cast<const ET*>(raw);
    if (bounded)
        gate_transform_kernel<ET, true><<<grid, 256, 0, s>>>(r, A_log, dt_bias, n, H, D, lb, out);
    else
        gate_transform_kernel<ET, false><<<grid, 256, 0, s>>>(r, A_log, dt_bias, n, H, D, lb, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_transform(bool bf16, bool bounded, const void* raw, const float* A_log, const float* dt_bias,
                                 long n, int H, int D, float lower_bound, float* out, hipStream_t s) {
    if (n == 0) return hipSuccess;
    timing_begin("gate_transform", s);
    const hipError_t e = bf16 ? launch_typed<bf16_t>(bounded, raw, A_log, dt_bias, n, H, D, lower_bound, out, s)
                              : launch_typed<float>(bounded, raw, A_log, dt_bias, n, H, D, lower_bound, out, s);
    timing_end(s);
    return e;
}

}  // namespace sf

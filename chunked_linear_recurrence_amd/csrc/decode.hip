// One-token paged Gated Delta Rule decode for gfx950.
//
// attention-gym "Linear Attention": the recurrent_gdn_decode entry (one token per sequence, the
// packed post-convolution row [Q heads | K heads | V heads], grouped q/k heads, an FP32 or BF16
// state pool [num_slots, H, V, K] advanced in place through per-sequence slot indices, null
// slots, a fresh-slot mask) and the section "Gate Transforms" (softplus convention). Per
// (sequence b, value head h), in float32:
//
//   q^ = q / sqrt(|q|^2 + 1e-6),  k^ likewise           (q, k of q/k head h / (H / HK))
//   g = -exp(A_log[h]) softplus(raw_gate + dt_bias[h]),  beta = sigmoid(raw_beta)
//   S = pool[slot, h]  (zero for a fresh slot)
//   S <- exp(g) S;  r = beta (v - S k^);  S <- S + r k^T;  o = scale S q^
//   pool[slot, h] = S,  out[b, h] = o
//
// The state is read once and written once, so the kernel is bound by HBM: a workgroup of four
// wavefronts owns one (sequence, head); lane groups of K/4 lanes hold one state row, four
// consecutive key columns per lane (16-byte loads and stores of the float32 pool), and the two
// row sums (S k^ and S q^) are butterfly sums over the group. Eight row iterations of loads are
// issued before any arithmetic so that each wavefront keeps 8 KB in flight.
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {
namespace {

constexpr float kL2Eps = 1e-6f;
constexpr int kDecodeWaves = 4;
constexpr int kDecodeBatch = 8;  // row iterations whose loads are issued together

template <typename T> struct Io;
template <> struct Io<float> {
    static __device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ void store4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
    static __device__ __forceinline__ float load1(const float* p) { return *p; }
    static __device__ __forceinline__ void store1(float* p, float x) { *p = x; }
};
template <> struct Io<bf16_t> {
    static __device__ __forceinline__ f32x4 load4(const bf16_t* p) {
        return Elem<bf16_t>::unpack(*reinterpret_cast<const i16x4*>(p));
    }
    static __device__ __forceinline__ void store4(bf16_t* p, f32x4 x) {
        *reinterpret_cast<i16x4*>(p) = Elem<bf16_t>::pack(x);
    }
    static __device__ __forceinline__ float load1(const bf16_t* p) { return bf2f(*p); }
    static __device__ __forceinline__ void store1(bf16_t* p, float x) { *p = f2bf(x); }
};

// sum over the LPR consecutive lanes of one row group (LPR a power of two dividing 64)
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = LPR / 2; m > 0; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

template <typename ET, typename PT, int K>
__global__ __launch_bounds__(64 * kDecodeWaves) void gdn_decode_kernel(
    const ET* __restrict__ qkv, const ET* __restrict__ raw_gate, const ET* __restrict__ raw_beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, PT* __restrict__ pool,
    long long slot_stride, int num_slots, const int32_t* __restrict__ state_indices,
    const uint8_t* __restrict__ has_init, int H, int HK, int V, float scale, ET* __restrict__ out) {
    constexpr int LPR = K / 4;      // lanes per state row
    constexpr int RPI = 64 / LPR;   // rows per wavefront instruction
    const int b = blockIdx.x / H, h = blockIdx.x - b * H;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int slot = state_indices[b];
    ET* o = out + ((size_t)b * H + h) * V;
    if (slot <= 0 || slot >= num_slots) {  // null row (or an index past the pool): zero output, no state traffic
        for (int r = threadIdx.x; r < V; r += 64 * kDecodeWaves) Io<ET>::store1(o + r, 0.f);
        return;
    }
    const int hk = h / (H / HK);
    const ET* x = qkv + (size_t)b * ((size_t)2 * HK * K + (size_t)H * V);
    const int c0 = 4 * (lane % LPR), rin = lane / LPR;

    // normalised q and k columns c0..c0+3 (every row group holds the same copy)
    f32x4 qv = Io<ET>::load4(x + hk * K + c0);
    f32x4 kv = Io<ET>::load4(x + (size_t)HK * K + hk * K + c0);
    qv = qv * (1.f / sqrtf(group_sum<LPR>(dot4(qv, qv)) + kL2Eps));
    kv = kv * (1.f / sqrtf(group_sum<LPR>(dot4(kv, kv)) + kL2Eps));
    // gates: softplus(a) = max(a, 0) + log(1 + exp(-|a|)) never overflows
    const float a = Io<ET>::load1(raw_gate + (size_t)b * H + h) + dt_bias[h];
    const float sp = fmaxf(a, 0.f) + log1pf(expf(-fabsf(a)));
    const float gamma = expf(-expf(A_log[h]) * sp);
    const float beta = 1.f / (1.f + expf(-Io<ET>::load1(raw_beta + (size_t)b * H + h)));
    const bool init = has_init == nullptr || has_init[b] != 0;

    const ET* vrow = x + (size_t)2 * HK * K + (size_t)h * V;
    PT* S0 = pool + (size_t)slot * (size_t)slot_stride + (size_t)h * V * K;
    const int rows_w = V / kDecodeWaves, nit = rows_w / RPI;
    for (int i0 = 0; i0 < nit; i0 += kDecodeBatch) {
        f32x4 S[kDecodeBatch];
        float vv[kDecodeBatch];
#pragma unroll
        for (int j = 0; j < kDecodeBatch; ++j) {
            if (i0 + j < nit) {
                const int row = w * rows_w + (i0 + j) * RPI + rin;
                S[j] = init ? Io<PT>::load4(S0 + (size_t)row * K + c0) : f32x4{0.f, 0.f, 0.f, 0.f};
                vv[j] = Io<ET>::load1(vrow + row);
            }
        }
#pragma unroll
        for (int j = 0; j < kDecodeBatch; ++j) {
            if (i0 + j < nit) {  // uniform over the wavefront: the group sums run on full lanes
                const int row = w * rows_w + (i0 + j) * RPI + rin;
                const float r = beta * (vv[j] - gamma * group_sum<LPR>(dot4(S[j], kv)));
                const f32x4 Sn = S[j] * gamma + kv * r;
                const float ov = group_sum<LPR>(dot4(Sn, qv));
                Io<PT>::store4(S0 + (size_t)row * K + c0, Sn);
                if (lane % LPR == 0) Io<ET>::store1(o + row, scale * ov);
            }
        }
    }
}

template <typename ET, typename PT>
hipError_t launch_typed(int K, const void* qkv, const void* rg, const void* rb, const float* A_log,
                        const float* dt_bias, void* pool, long long slot_stride, int num_slots,
                        const int32_t* idx, const uint8_t* has_init, int B, int H, int HK, int V,
                        float scale, void* out, hipStream_t s) {
    const dim3 grid((unsigned)B * (unsigned)H), block(64 * kDecodeWaves);
    const ET* q = static_cast<const ET*>(qkv);
    const ET* g = static_cast<const ET*>(rg);
    const ET* bt = static_cast<const ET*>(rb);
    PT* p = static_cast<PT*>(pool);
    ET* o = static_cast<ET*>(out);
    if (K == 64)
        gdn_decode_kernel<ET, PT, 64><<<grid, block, 0, s>>>(q, g, bt, A_log, dt_bias, p, slot_stride, num_slots, idx,
                                                             has_init, H, HK, V, scale, o);
    else if (K == 128)
        gdn_decode_kernel<ET, PT, 128><<<grid, block, 0, s>>>(q, g, bt, A_log, dt_bias, p, slot_stride, num_slots, idx,
                                                              has_init, H, HK, V, scale, o);
    else
        gdn_decode_kernel<ET, PT, 256><<<grid, block, 0, s>>>(q, g, bt, A_log, dt_bias, p, slot_stride, num_slots, idx,
                                                              has_init, H, HK, V, scale, o);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gdn_decode(bool bf16, bool pool_bf16, const void* qkv, const void* raw_gate,
                             const void* raw_beta, const float* A_log, const float* dt_bias, void* pool,
                             long long slot_stride, int num_slots, const int32_t* state_indices,
                             const uint8_t* has_init, int B, int H, int HK, int K, int V, float scale,
                             void* out, hipStream_t s) {
    if (B == 0) return hipSuccess;
    timing_begin("gdn_decode", s);
    hipError_t e;
    if (bf16)
        e = pool_bf16 ? launch_typed<bf16_t, bf16_t>(K, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                                     num_slots, state_indices, has_init, B, H, HK, V, scale, out, s)
                      : launch_typed<bf16_t, float>(K, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                                    num_slots, state_indices, has_init, B, H, HK, V, scale, out, s);
    else
        e = pool_bf16 ? launch_typed<float, bf16_t>(K, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                                    num_slots, state_indices, has_init, B, H, HK, V, scale, out, s)
                      : launch_typed<float, float>(K, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                                   num_slots, state_indices, has_init, B, H, HK, V, scale, out, s);
    timing_end(s);
    return e;
}

}  // namespace sf

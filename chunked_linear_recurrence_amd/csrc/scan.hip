// Exclusive scan of segment summaries (Megatron-LM "Mamba2 state-passing
// context parallelism": exclusive causal scan over per-segment summaries;
// attention-gym "Context Parallelism": composition of affine range maps).
//
//   S_in[j = 0]   = h0 (or zeros)
//   S_in[j + 1]   = S_in[j] @ M[j] + S_ext[j]    delta rule, M [K x K]
//                 = a[j] S_in[j] + S_ext[j]      scalar gate
//   S_final       = the step after the last segment
//
// Delta rule: one workgroup per (batch row, head, 16 state rows). The 16 x K
// slice of the running state lives in LDS in float32; each step is a
// [16 x K] @ [K x K] float32 MFMA product (v_mfma_f32_16x16x4_f32), the
// four wavefronts splitting the output columns. A step's M and S_ext
// fragments are loaded during the step before.
// Scalar gate: elementwise, one thread per four state elements.
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {

template <int KD>
__global__ __launch_bounds__(256) void gdn_scan_kernel(const float* __restrict__ M,
                                                       const float* __restrict__ E,
                                                       const float* __restrict__ h0, int n_seg, int H,
                                                       int V, float* __restrict__ S_in,
                                                       float* __restrict__ S_final) {
    constexpr int LD = KD + 4;
    constexpr int NTW = KD / 16 / 4;  // output column tiles per wavefront
    constexpr int KBN = KD / 16;      // 16-row blocks of M
    __shared__ __align__(16) float sS[16 * LD];
    const int nvs = V / 16;
    const int vs = blockIdx.x % nvs, h = (blockIdx.x / nvs) % H, b = blockIdx.x / (nvs * H);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int r0 = vs * 16;
    const size_t VK = (size_t)V * KD;

    // Operands of step j (this wavefront's column tiles): the B fragments of M_j and the S_ext_j
    // tile that starts the accumulator. They do not depend on the running state, so step j+1's are
    // loaded while step j's products run.
    typedef f32x4 StepM[NTW][KBN];
    typedef f32x4 StepE[NTW];
    auto load_step = [&](int j, StepM& bm, StepE& e) __attribute__((always_inline)) {
        const size_t sh = ((size_t)(b * n_seg + j) * H + h);
        const float* Mj = M + sh * KD * KD;
        const float* Ej = E + sh * VK;
#pragma unroll
        for (int w = 0; w < NTW; ++w) {
            const int n0 = (wave * NTW + w) * 16;
#pragma unroll
            for (int r = 0; r < 4; ++r) e[w][r] = Ej[(size_t)(r0 + 4 * lg + r) * KD + n0 + ln];
#pragma unroll
            for (int kb = 0; kb < KBN; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) bm[w][kb][r] = Mj[(size_t)(16 * kb + 4 * lg + r) * KD + n0 + ln];
        }
    };

    for (int i = tid; i < 16 * KD; i += 256) {
        const int r = i / KD, c = i % KD;
        sS[r * LD + c] = h0 ? h0[((size_t)b * H + h) * VK + (size_t)(r0 + r) * KD + c] : 0.f;
    }
    StepM bm;
    StepE e;
    if (n_seg > 0) load_step(0, bm, e);
    for (int j = 0; j < n_seg; ++j) {
        StepM bmn;
        StepE en;
        if (j + 1 < n_seg) load_step(j + 1, bmn, en);
        const size_t sh = ((size_t)(b * n_seg + j) * H + h);
        __syncthreads();
        for (int i = tid; i < 16 * KD; i += 256) {
            const int r = i / KD, c = i % KD;
            S_in[sh * VK + (size_t)(r0 + r) * KD + c] = sS[r * LD + c];
        }
        f32x4 acc[NTW];
#pragma unroll
        for (int w = 0; w < NTW; ++w) {
            acc[w] = e[w];
#pragma unroll
            for (int kb = 0; kb < KBN; ++kb) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(&sS[ln * LD + 16 * kb + 4 * lg]);
                acc[w] = Elem<float>::mma(acc[w], a, bm[w][kb]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NTW; ++w) {
            const int n0 = (wave * NTW + w) * 16;
#pragma unroll
            for (int r = 0; r < 4; ++r) sS[(4 * lg + r) * LD + n0 + ln] = acc[w][r];
        }
        if (j + 1 < n_seg) {
#pragma unroll
            for (int w = 0; w < NTW; ++w) {
                e[w] = en[w];
#pragma unroll
                for (int kb = 0; kb < KBN; ++kb) bm[w][kb] = bmn[w][kb];
            }
        }
    }
    __syncthreads();
    if (S_final) {
        for (int i = tid; i < 16 * KD; i += 256) {
            const int r = i / KD, c = i % KD;
            S_final[((size_t)b * H + h) * VK + (size_t)(r0 + r) * KD + c] = sS[r * LD + c];
        }
    }
}

__global__ __launch_bounds__(256) void gla_scan_kernel(const float* __restrict__ a,
                                                       const float* __restrict__ E,
                                                       const float* __restrict__ h0, int B, int n_seg,
                                                       int H, int VK, float* __restrict__ S_in,
                                                       float* __restrict__ S_final) {
    const size_t per_b = (size_t)H * VK;
    const size_t i4 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= (size_t)B * per_b) return;
    const int b = (int)(i4 / per_b);
    const size_t rem = i4 % per_b;
    const int h = (int)(rem / VK);
    f32x4 cur = h0 ? *reinterpret_cast<const f32x4*>(h0 + i4) : zero4();
    for (int j = 0; j < n_seg; ++j) {
        const size_t s = (size_t)b * n_seg + j;
        *reinterpret_cast<f32x4*>(S_in + s * per_b + rem) = cur;
        const float aj = a[s * H + h];
        const f32x4 e = *reinterpret_cast<const f32x4*>(E + s * per_b + rem);
        cur = cur * aj + e;
    }
    if (S_final) *reinterpret_cast<f32x4*>(S_final + i4) = cur;
}

hipError_t launch_scan(int kind, const float* M, const float* S_ext, const float* h0, int B,
                       int n_seg, int H, int K, int V, float* S_in, float* S_final, hipStream_t s) {
    if (kind == 0) {
        const unsigned grid = (unsigned)B * H * (V / 16);
        if (grid == 0) return hipSuccess;
        timing_begin("gdn_state_scan", s);
        if (K == 128)
            gdn_scan_kernel<128><<<grid, 256, 0, s>>>(M, S_ext, h0, n_seg, H, V, S_in, S_final);
        else
            gdn_scan_kernel<64><<<grid, 256, 0, s>>>(M, S_ext, h0, n_seg, H, V, S_in, S_final);
    } else {
        const size_t n4 = (size_t)B * H * V * K / 4;
        if (n4 == 0) return hipSuccess;
        timing_begin("gla_state_scan", s);
        gla_scan_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(M, S_ext, h0, B, n_seg, H, V * K, S_in, S_final);
    }
    timing_end(s);
    return hipGetLastError();
}

}  // namespace sf

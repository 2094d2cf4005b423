// Token-by-token Gated Delta Rule kernels for gfx950: the one-token paged decode and the
// multi-token recurrent forward.
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
//
// Recurrent forward (attention-gym "Linear Attention", the recurrent_gdn entry): the same token
// rule over a whole sequence, with g and beta as given and q, k used as given. The state stays
// in registers from the first token to the last: a workgroup of four wavefronts owns 32 state
// rows of one (sequence, head), eight lanes per row with K/8 consecutive key columns each, so
// each row sum is a lane's own dot product plus three DPP lane permutations. The token operands
// (q, k, the 32 values, the two gates) come in blocks of 16 tokens: the workgroup loads the next
// block into registers while it computes the current one, then widens it to float32 in LDS once
// for all 32 rows, so a token step waits on LDS, not on memory, and converts nothing; outputs
// leave once per block, one row piece per token and wavefront.
// The state comes from h0 (or zero) and goes to ht, or, with slot indices, from and back to a
// paged pool.
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

// CH: Kimi Delta Attention (recurrent_kda_decode): raw_gate [B, H, K] and dt_bias [H, K] per key
// channel through the bounded (lower_bound sigmoid(exp(A_log) a)) or softplus kind, each key column
// decayed by its own factor; without CH the per-head softplus gate of the delta rule.
template <typename ET, typename PT, int K, bool CH>
__global__ __launch_bounds__(64 * kDecodeWaves) void gdn_decode_kernel(
    const ET* __restrict__ qkv, const ET* __restrict__ raw_gate, const ET* __restrict__ raw_beta,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias, PT* __restrict__ pool,
    long long slot_stride, int num_slots, const int32_t* __restrict__ state_indices,
    const uint8_t* __restrict__ has_init, int H, int HK, int V, float scale, ET* __restrict__ out, int bounded,
    float lower_bound) {
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
    float gamma = 1.f;
    f32x4 alpha = {1.f, 1.f, 1.f, 1.f};  // per-channel decay of columns c0..c0+3 (CH)
    if constexpr (CH) {
        const f32x4 a = Io<ET>::load4(raw_gate + ((size_t)b * H + h) * K + c0) +
                        *reinterpret_cast<const f32x4*>(dt_bias + (size_t)h * K + c0);
        const float amp = expf(A_log[h]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            alpha[e] = expf(bounded ? lower_bound / (1.f + expf(-amp * a[e]))
                                    : -amp * (fmaxf(a[e], 0.f) + log1pf(expf(-fabsf(a[e])))));
    } else {
        const float a = Io<ET>::load1(raw_gate + (size_t)b * H + h) + dt_bias[h];
        gamma = expf(-expf(A_log[h]) * (fmaxf(a, 0.f) + log1pf(expf(-fabsf(a)))));
    }
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
                const f32x4 Sd = CH ? S[j] * alpha : S[j];  // (the scalar decay is folded in below)
                const float r = beta * (vv[j] - gamma * group_sum<LPR>(dot4(Sd, kv)));
                const f32x4 Sn = CH ? Sd + kv * r : S[j] * gamma + kv * r;
                const float ov = group_sum<LPR>(dot4(Sn, qv));
                Io<PT>::store4(S0 + (size_t)row * K + c0, Sn);
                if (lane % LPR == 0) Io<ET>::store1(o + row, scale * ov);
            }
        }
    }
}

constexpr int kRecLpr = 8;     // lanes per state row in the recurrent kernel
constexpr int kRecWaves = 4;   // wavefronts per recurrent workgroup
constexpr int kRecRows = kRecWaves * 64 / kRecLpr;  // state rows per workgroup (32)
constexpr int kRecTok = 16;    // tokens per block staged in LDS

// raw (unconverted) four-element vectors of the token operands
template <typename T> struct Raw;
template <> struct Raw<float> {
    typedef f32x4 type;
    static __device__ __forceinline__ type load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ f32x4 cvt(type x) { return x; }
};
template <> struct Raw<bf16_t> {
    typedef i16x4 type;
    static __device__ __forceinline__ type load(const bf16_t* p) { return *reinterpret_cast<const i16x4*>(p); }
    static __device__ __forceinline__ f32x4 cvt(type x) { return Elem<bf16_t>::unpack(x); }
};

// sum over the eight lanes of a row group with DPP: quad permutations (lane i reads lane i^1, then
// i^2), then the half-row mirror (lane i reads lane 7-i of its eight)
// (every source lane exists, so bound_ctrl changes nothing and lets each move fold into its add)
__device__ __forceinline__ float row_group_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
    return x;
}

// a + x . y as four fused multiply-adds
__device__ __forceinline__ float fma4(f32x4 x, f32x4 y, float a) {
    return fmaf(x[3], y[3], fmaf(x[2], y[2], fmaf(x[1], y[1], fmaf(x[0], y[0], a))));
}

// LDS plan of one recurrent workgroup: one token block, widened to float32 once for all rows
// (CH: per-channel gates, whose decay factors exp(g) take one more [16][K] block)
template <int K, bool CH>
struct RecLds {
    static constexpr int OFF_Q = 0;                                  // float [16][K]
    static constexpr int OFF_K = OFF_Q + kRecTok * K * 4;            // float [16][K]
    static constexpr int OFF_A = OFF_K + kRecTok * K * 4;            // float [16][K] exp(g) (CH only)
    static constexpr int OFF_V = OFF_A + (CH ? kRecTok * K * 4 : 0); // float [16][32]
    static constexpr int OFF_G = OFF_V + kRecTok * kRecRows * 4;     // float g[16], beta[16]
    static constexpr int OFF_O = OFF_G + 2 * kRecTok * 4;            // float outputs [wave][16][8]
    static constexpr int BYTES = OFF_O + kRecWaves * kRecTok * 8 * 4;
};

template <typename ET, typename PT, int K, bool CH>
__global__ __launch_bounds__(64 * kRecWaves) void gdn_recurrent_kernel(
    const ET* __restrict__ q, const ET* __restrict__ k, const ET* __restrict__ v, const float* __restrict__ g,
    const float* __restrict__ beta, const float* __restrict__ h0, float* __restrict__ ht, PT* __restrict__ pool,
    long long slot_stride, int num_slots, const int32_t* __restrict__ state_indices,
    const uint8_t* __restrict__ has_init, const int32_t* __restrict__ cu, int T, int H, int HK, int V, float scale,
    ET* __restrict__ out, int n_pairs) {
    typedef RecLds<K, CH> SM;
    constexpr int CPL = K / kRecLpr;  // key columns per lane: lanes 8r .. 8r+7 hold state row r of the wavefront
    constexpr int NV = CPL / 4;       // four-column vectors per lane
    constexpr int NT = 64 * kRecWaves;
    constexpr int NQ = kRecTok * K / 4 / NT;  // four-element q (and k) vectors each thread moves per block
    static_assert(NQ >= 1 && kRecTok * K % (4 * NT) == 0, "block split");
    typedef typename Raw<ET>::type RawT;
    __shared__ __align__(16) uint8_t smem[SM::BYTES];
    typedef __attribute__((address_space(3))) float lds_f;
    typedef __attribute__((address_space(3))) f32x4 lds_f4;
    lds_f* const sQ = (lds_f*)(smem + SM::OFF_Q);
    lds_f* const sK = (lds_f*)(smem + SM::OFF_K);
    lds_f* const sA = (lds_f*)(smem + SM::OFF_A);
    lds_f* const sV = (lds_f*)(smem + SM::OFF_V);
    lds_f* const sG = (lds_f*)(smem + SM::OFF_G);

    // the nvb workgroups of one (sequence, head) share its q and k: they run on one XCD (whose L2
    // then fetches those rows once); workgroups past the last pair of a padded grid exit
    const int nvb = V / kRecRows;
    int nh, vb;
    xcd_split(blockIdx.x, nvb, nh, vb);
    if (nh >= n_pairs) return;
    const int n = nh / H, h = nh - n * H, hk = h / (H / HK);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int rl = 8 * w + lane / kRecLpr;     // row within the workgroup's 32
    const int r0 = kRecRows * vb, row = r0 + rl;
    const int c0 = CPL * (lane % kRecLpr);
    int b, bos, eos;
    if (cu) {
        b = 0;
        bos = cu[n];
        eos = cu[n + 1];
    } else {
        b = n;
        bos = 0;
        eos = T;
    }
    PT* slot_p = nullptr;
    if (pool) {
        const int slot = state_indices[n];
        if (slot <= 0 || slot >= num_slots) {  // null sequence: zero output rows, no state access
            for (int t = bos + tid / kRecRows; t < eos; t += NT / kRecRows)
                Io<ET>::store1(out + ((size_t)(b * T + t) * H + h) * V + r0 + tid % kRecRows, 0.f);
            return;
        }
        slot_p = pool + (size_t)slot * (size_t)slot_stride + (size_t)h * V * K;
    }
    const float* h0p = h0 ? h0 + ((size_t)n * H + h) * V * K : nullptr;
    float* htp = ht ? ht + ((size_t)n * H + h) * V * K : nullptr;
    const bool load_slot = slot_p && (has_init == nullptr || has_init[n] != 0);
    const size_t soff = (size_t)row * K + c0;

    f32x4 S[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        S[i] = load_slot ? Io<PT>::load4(slot_p + soff + 4 * i)
                         : (h0p ? Io<float>::load4(h0p + soff + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f});

    // one token block [t0, t0 + 16) into registers: thread tid moves q and k vectors tid + 256 i,
    // two values and (threads 0..31) one gate; tokens past the end repeat the last token (their
    // results are never stored)
    struct Blk {
        RawT q[NQ], k[NQ];
        f32x4 a[CH ? NQ : 1];  // per-channel gates (CH)
        float v0, v1, gb;
    };
    auto fetch = [&](int t0, Blk& x) __attribute__((always_inline)) {
        const int last = eos - 1;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int e = 4 * (tid + NT * i), tt = min(t0 + e / K, last);
            const size_t src = ((size_t)(b * T + tt) * HK + hk) * K + e % K;
            x.q[i] = Raw<ET>::load(q + src);
            x.k[i] = Raw<ET>::load(k + src);
            if constexpr (CH) x.a[i] = *reinterpret_cast<const f32x4*>(g + ((size_t)(b * T + tt) * H + h) * K + e % K);
        }
        const int tv = min(t0 + tid / 16, last), rv = 2 * (tid % 16);
        const ET* vp = v + ((size_t)(b * T + tv) * H + h) * V + r0 + rv;
        x.v0 = Io<ET>::load1(vp);
        x.v1 = Io<ET>::load1(vp + 1);
        x.gb = 0.f;
        if (tid < 2 * kRecTok && (!CH || tid >= kRecTok))
            x.gb = (tid < kRecTok ? g : beta)[(size_t)(b * T + min(t0 + tid % kRecTok, last)) * H + h];
    };
    auto stage = [&](const Blk& x) __attribute__((always_inline)) {  // widen into LDS
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            *(lds_f4*)(sQ + 4 * (tid + NT * i)) = Raw<ET>::cvt(x.q[i]);
            *(lds_f4*)(sK + 4 * (tid + NT * i)) = Raw<ET>::cvt(x.k[i]);
            if constexpr (CH) {
                f32x4 d;
#pragma unroll
                for (int e = 0; e < 4; ++e) d[e] = expf(x.a[i][e]);
                *(lds_f4*)(sA + 4 * (tid + NT * i)) = d;
            }
        }
        sV[2 * tid] = x.v0;
        sV[2 * tid + 1] = x.v1;
        if (tid < 2 * kRecTok) sG[tid] = x.gb;
    };
    const int nblk = (eos - bos + kRecTok - 1) / kRecTok;
    Blk nb;
    if (nblk > 0) fetch(bos, nb);
    lds_f* const obuf = (lds_f*)(smem + SM::OFF_O) + w * (kRecTok * 8);
    for (int blk = 0; blk < nblk; ++blk) {
        const int t0 = bos + blk * kRecTok, nt = min(kRecTok, eos - t0);
        __syncthreads();  // every wavefront is done with the previous block's LDS
        stage(nb);
        if (blk + 1 < nblk) fetch(t0 + kRecTok, nb);
        __syncthreads();  // the block is in LDS
        for (int tt = 0; tt < nt; ++tt) {
            const lds_f* qr = sQ + tt * K + c0;
            const lds_f* kr = sK + tt * K + c0;
            const float bt = sG[kRecTok + tt], vv = sV[tt * kRecRows + rl];
            float gamma = 1.f;
            if constexpr (CH) {  // decay each key column by its own factor first
                const lds_f* ar = sA + tt * K + c0;
#pragma unroll
                for (int i = 0; i < NV; ++i) S[i] = S[i] * *(const lds_f4*)(ar + 4 * i);
            } else {
                gamma = expf(sG[tt]);
            }
            f32x4 kf[NV];
            float sk0 = 0.f, sk1 = 0.f;  // two accumulation chains
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                kf[i] = *(const lds_f4*)(kr + 4 * i);
                if (i & 1)
                    sk1 = fma4(S[i], kf[i], sk1);
                else
                    sk0 = fma4(S[i], kf[i], sk0);
            }
            const float r = bt * (vv - gamma * row_group_sum(sk0 + sk1));
            float so0 = 0.f, so1 = 0.f;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) S[i][e] = CH ? fmaf(kf[i][e], r, S[i][e]) : fmaf(kf[i][e], r, S[i][e] * gamma);
                if (i & 1)
                    so1 = fma4(S[i], *(const lds_f4*)(qr + 4 * i), so1);
                else
                    so0 = fma4(S[i], *(const lds_f4*)(qr + 4 * i), so0);
            }
            const float so = row_group_sum(so0 + so1);
            if (lane % kRecLpr == 0) obuf[tt * 8 + lane / kRecLpr] = scale * so;
        }
        // the wavefront's 8 outputs of each token of the block: one row piece per lane
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane < nt) {
            ET* dst = out + ((size_t)(b * T + t0 + lane) * H + h) * V + r0 + 8 * w;
            const f32x4 lo = *(const lds_f4*)(obuf + 8 * lane), hi = *(const lds_f4*)(obuf + 8 * lane + 4);
            Io<ET>::store4(dst, lo);
            Io<ET>::store4(dst + 4, hi);
        }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (slot_p)
            Io<PT>::store4(slot_p + soff + 4 * i, S[i]);
        else if (htp)
            Io<float>::store4(htp + soff + 4 * i, S[i]);
    }
}

template <typename ET, typename PT, bool CH>
hipError_t launch_rec_typed(int K, const void* q, const void* k, const void* v, const float* g, const float* beta,
                            const float* h0, float* ht, void* pool, long long slot_stride, int num_slots,
                            const int32_t* idx, const uint8_t* has_init, const int32_t* cu, int N, int T, int H,
                            int HK, int V, float scale, void* out, hipStream_t s) {
    const unsigned pairs = (unsigned)N * (unsigned)H;
    const dim3 grid(((pairs + 7) / 8) * 8 * (unsigned)(V / kRecRows)), block(64 * kRecWaves);
    const ET *qq = static_cast<const ET*>(q), *kk = static_cast<const ET*>(k), *vv = static_cast<const ET*>(v);
    PT* p = static_cast<PT*>(pool);
    ET* o = static_cast<ET*>(out);
    if (K == 64)
        gdn_recurrent_kernel<ET, PT, 64, CH><<<grid, block, 0, s>>>(qq, kk, vv, g, beta, h0, ht, p, slot_stride, num_slots,
                                                                idx, has_init, cu, T, H, HK, V, scale, o, (int)pairs);
    else if (K == 128)
        gdn_recurrent_kernel<ET, PT, 128, CH><<<grid, block, 0, s>>>(qq, kk, vv, g, beta, h0, ht, p, slot_stride,
                                                                 num_slots, idx, has_init, cu, T, H, HK, V, scale, o, (int)pairs);
    else
        gdn_recurrent_kernel<ET, PT, 256, CH><<<grid, block, 0, s>>>(qq, kk, vv, g, beta, h0, ht, p, slot_stride,
                                                                 num_slots, idx, has_init, cu, T, H, HK, V, scale, o, (int)pairs);
    return hipGetLastError();
}

template <typename ET, typename PT, bool CH>
hipError_t launch_typed(int K, const void* qkv, const void* rg, const void* rb, const float* A_log,
                        const float* dt_bias, void* pool, long long slot_stride, int num_slots,
                        const int32_t* idx, const uint8_t* has_init, int B, int H, int HK, int V,
                        float scale, void* out, hipStream_t s, int bounded, float lb) {
    const dim3 grid((unsigned)B * (unsigned)H), block(64 * kDecodeWaves);
    const ET* q = static_cast<const ET*>(qkv);
    const ET* g = static_cast<const ET*>(rg);
    const ET* bt = static_cast<const ET*>(rb);
    PT* p = static_cast<PT*>(pool);
    ET* o = static_cast<ET*>(out);
    if (K == 64)
        gdn_decode_kernel<ET, PT, 64, CH><<<grid, block, 0, s>>>(q, g, bt, A_log, dt_bias, p, slot_stride, num_slots, idx,
                                                             has_init, H, HK, V, scale, o, bounded, lb);
    else if (K == 128)
        gdn_decode_kernel<ET, PT, 128, CH><<<grid, block, 0, s>>>(q, g, bt, A_log, dt_bias, p, slot_stride, num_slots, idx,
                                                              has_init, H, HK, V, scale, o, bounded, lb);
    else
        gdn_decode_kernel<ET, PT, 256, CH><<<grid, block, 0, s>>>(q, g, bt, A_log, dt_bias, p, slot_stride, num_slots, idx,
                                                              has_init, H, HK, V, scale, o, bounded, lb);
    return hipGetLastError();
}

}  // namespace

template <bool CH>
hipError_t launch_rec(bool bf16, bool pool_bf16, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, const float* h0, float* ht, void* pool, long long slot_stride, int num_slots,
                      const int32_t* state_indices, const uint8_t* has_init, const int32_t* cu, int N, int T, int H,
                      int HK, int K, int V, float scale, void* out, hipStream_t s) {
    if (bf16)
        return pool_bf16 ? launch_rec_typed<bf16_t, bf16_t, CH>(K, q, k, v, g, beta, h0, ht, pool, slot_stride, num_slots,
                                                                state_indices, has_init, cu, N, T, H, HK, V, scale, out, s)
                         : launch_rec_typed<bf16_t, float, CH>(K, q, k, v, g, beta, h0, ht, pool, slot_stride, num_slots,
                                                               state_indices, has_init, cu, N, T, H, HK, V, scale, out, s);
    return pool_bf16 ? launch_rec_typed<float, bf16_t, CH>(K, q, k, v, g, beta, h0, ht, pool, slot_stride, num_slots,
                                                           state_indices, has_init, cu, N, T, H, HK, V, scale, out, s)
                     : launch_rec_typed<float, float, CH>(K, q, k, v, g, beta, h0, ht, pool, slot_stride, num_slots,
                                                          state_indices, has_init, cu, N, T, H, HK, V, scale, out, s);
}

hipError_t launch_gdn_recurrent(bool bf16, bool pool_bf16, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, const float* h0, float* ht, void* pool,
                                long long slot_stride, int num_slots, const int32_t* state_indices,
                                const uint8_t* has_init, const int32_t* cu, int N, int T, int H, int HK, int K,
                                int V, float scale, void* out, hipStream_t s, bool per_channel) {
    if (N == 0) return hipSuccess;
    timing_begin(per_channel ? "kda_recurrent" : "gdn_recurrent", s);
    const hipError_t e = per_channel
        ? launch_rec<true>(bf16, pool_bf16, q, k, v, g, beta, h0, ht, pool, slot_stride, num_slots, state_indices,
                           has_init, cu, N, T, H, HK, K, V, scale, out, s)
        : launch_rec<false>(bf16, pool_bf16, q, k, v, g, beta, h0, ht, pool, slot_stride, num_slots, state_indices,
                            has_init, cu, N, T, H, HK, K, V, scale, out, s);
    timing_end(s);
    return e;
}

template <bool CH>
hipError_t launch_dec(bool bf16, bool pool_bf16, const void* qkv, const void* raw_gate, const void* raw_beta,
                      const float* A_log, const float* dt_bias, void* pool, long long slot_stride, int num_slots,
                      const int32_t* idx, const uint8_t* has_init, int B, int H, int HK, int K, int V, float scale,
                      void* out, hipStream_t s, int bounded, float lb) {
    if (bf16)
        return pool_bf16 ? launch_typed<bf16_t, bf16_t, CH>(K, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                                            num_slots, idx, has_init, B, H, HK, V, scale, out, s, bounded, lb)
                         : launch_typed<bf16_t, float, CH>(K, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                                           num_slots, idx, has_init, B, H, HK, V, scale, out, s, bounded, lb);
    return pool_bf16 ? launch_typed<float, bf16_t, CH>(K, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                                       num_slots, idx, has_init, B, H, HK, V, scale, out, s, bounded, lb)
                     : launch_typed<float, float, CH>(K, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                                      num_slots, idx, has_init, B, H, HK, V, scale, out, s, bounded, lb);
}

hipError_t launch_gdn_decode(bool bf16, bool pool_bf16, const void* qkv, const void* raw_gate,
                             const void* raw_beta, const float* A_log, const float* dt_bias, void* pool,
                             long long slot_stride, int num_slots, const int32_t* state_indices,
                             const uint8_t* has_init, int B, int H, int HK, int K, int V, float scale,
                             void* out, hipStream_t s, bool per_channel, int bounded, float lower_bound) {
    if (B == 0) return hipSuccess;
    timing_begin(per_channel ? "kda_decode" : "gdn_decode", s);
    const hipError_t e =
        per_channel ? launch_dec<true>(bf16, pool_bf16, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                       num_slots, state_indices, has_init, B, H, HK, K, V, scale, out, s, bounded,
                                       lower_bound)
                    : launch_dec<false>(bf16, pool_bf16, qkv, raw_gate, raw_beta, A_log, dt_bias, pool, slot_stride,
                                        num_slots, state_indices, has_init, B, H, HK, K, V, scale, out, s, 0, 0.f);
    timing_end(s);
    return e;
}

}  // namespace sf

// Kimi Delta Attention chunk forward for gfx950 (attention-gym "Linear Attention", section "Kimi Delta
// Attention", chunk_kda): the delta rule with a per-channel gate, run per 64-token chunk with the StateFlow
// Section 2.2, Eq. (2) split.
//
// For one chunk of one (sequence, head) with entry state S [V x K] and, per key channel c, the within-chunk
// cumulative gate G_t[c] = sum_{i<=t} g_i[c] (Gamma_t = exp(G_t), a vector over the channels), the token rule
// (the state decays channel by channel, then the delta rule's correction and update, then the read) unrolls to
//   A_ts = beta_t sum_c k_t[c] k_s[c] exp(G_t[c] - G_s[c])   (s < t),   T = (I + A)^-1,
//   W = T diag(beta) (Gamma o K),   U = T diag(beta) V,   R = U - W S^T,
//   P_ts = scale sum_c q_t[c] k_s[c] exp(G_t[c] - G_s[c])   (s <= t),   Qg = scale (Gamma o Q),
//   O = Qg S^T + P R,
//   S' = S diag(Gamma_L) + R^T Kh,   Kh_s = exp(G_L - G_s) o k_s,
// where o multiplies each token row by its channel vector. Every exponent above is <= 0 (the cumulative
// gate only falls within a chunk), so the chunk form is exact for any finite, nonpositive gate: the decay
// between two tokens is applied per pair and channel rather than factored through exp(+G), which can
// overflow float32 for strong gates.
//
// Kernels (float32 arithmetic; q, k, v and the output in the input type):
//   kda_prep_kernel   per (chunk, head): W, U, P, Qg, Kh and Gamma_L into a record
//   kda_chain_kernel  per (sequence, head, 16-row slice of the state): the state chain and the output
#include "f32_tiles.h"
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {
namespace {

constexpr int BC = kGdnChunk;
constexpr int NT = f32t::NT;
constexpr int NTP = 2 * NT;  // threads of the prep: eight wavefronts
using f32t::Tile;
using f32t::mm4;

// Record of one (chunk, head), floats: W [64][KD] | U [64][VD] | P [64][64] | Qg [64][KD] | Kh [64][KD] | Gamma_L [KD]
template <int KD>
struct KdaRec {
    static __host__ __device__ size_t w_off() { return 0; }
    static __host__ __device__ size_t u_off() { return (size_t)BC * KD; }
    static __host__ __device__ size_t p_off(int V) { return u_off() + (size_t)BC * V; }
    static __host__ __device__ size_t q_off(int V) { return p_off(V) + (size_t)BC * BC; }
    static __host__ __device__ size_t kh_off(int V) { return q_off(V) + (size_t)BC * KD; }
    static __host__ __device__ size_t gl_off(int V) { return kh_off(V) + (size_t)BC * KD; }
    static __host__ __device__ size_t floats(int V) { return gl_off(V) + KD; }
};

// Record of one (chunk, head) for bf16 input, bytes, inside the float32 record's footprint: W [64][KD] bf16 |
// Qg [64][KD] bf16 | Kh^T [KD][64] bf16 | P [64][64] bf16 | U [64][VD] float | Gamma_L [KD] float. The chain's
// products take bf16 operands, so the factors are stored as such (U stays float32: it enters R as it is).
template <int KD>
struct KdaRec16 {
    static constexpr size_t W_OFF = 0;
    static constexpr size_t Q_OFF = W_OFF + (size_t)BC * KD * 2;
    static constexpr size_t KT_OFF = Q_OFF + (size_t)BC * KD * 2;
    static constexpr size_t P_OFF = KT_OFF + (size_t)KD * BC * 2;
    static constexpr size_t U_OFF = P_OFF + (size_t)BC * BC * 2;
    static constexpr __host__ __device__ size_t gl_off(int V) { return U_OFF + (size_t)BC * V * 4; }
    static constexpr __host__ __device__ size_t bytes(int V) { return gl_off(V) + (size_t)KD * 4; }
};

// ---------------------------------------------------------------------------------------------------------
// Prep: per (chunk slot, head), wavefront w owning token rows 16 w .. 16 w + 15; float32 throughout.
//   G: the per-channel cumulative gate (one thread per channel).
//   A and P, block row w: the blocks left of the diagonal as float32 MFMA tiles, through the split
//     exp(G_t - G_s) = exp(G_t - G_r) exp(G_r - G_s) at the last token r of block w - 1 (s <= r < t, so both
//     factors are at most 1: no overflow for any nonpositive gate); the diagonal block with the pairwise
//     per-channel decays as they stand.
//   T = (I + A)^-1 by 16x16 blocks (the four diagonal blocks by column substitution, one wavefront each, then
//     T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj block diagonal by block diagonal).
//   W = T diag(beta) (Gamma o K) and U = T diag(beta) V as tiles; Qg, Kh and Gamma_L elementwise.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD, int VD>
__global__ __launch_bounds__(NTP) void kda_prep_kernel(const ST* __restrict__ q, const ST* __restrict__ k,
                                                      const ST* __restrict__ v, const float* __restrict__ g,
                                                      const float* __restrict__ beta, const int2* __restrict__ table,
                                                      const int32_t* __restrict__ cu, int T, int H, int nc, float scale,
                                                      float* __restrict__ rec) {
    typedef KdaRec<KD> RL;
    constexpr int LK = KD + 4, LL = BC + 1, LU = 17, NJ = KD / 16, NV = VD / 16;
    __shared__ __align__(16) float sK[BC * LK];
    __shared__ __align__(16) float sQ[BC * LK];
    __shared__ __align__(16) float sG[BC * LK];
    __shared__ float sA[BC * LL], sT[BC * LL], sP[BC * LL];
    __shared__ float sB[BC], sU[4 * 16 * LU];
    float* const sV = sQ;  // V rows (scaled by beta) replace Q rows once Qg is formed (VD <= KD)
    static_assert(VD <= KD, "V rows reuse the Q buffer");
    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const long row0 = (long)b * T + t0;
    Tile<ST, BC, VD, NTP> tv;  // V rows: loaded now, stored once the Q rows are no longer read
    {
        Tile<ST, BC, KD, NTP> tk, tq;
        Tile<float, BC, KD, NTP> tg;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tq.load(q + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tg.load(g + (row0 * H + h) * (long)KD, (long)H * KD, L);  // padded tokens: g = 0
        tv.load(v + (row0 * H + h) * (long)VD, (long)H * VD, L);
        tk.template store_rows<LK>(sK);
        tq.template store_rows<LK>(sQ);
        tg.template store_rows<LK>(sG);
    }
    if (tid < BC) sB[tid] = tid < L ? beta[(row0 + tid) * H + h] : 0.f;
    __syncthreads();
    // cumulative gate per channel, in place (the channel's 64 gates read into registers first)
    if (tid < KD) {
        float gv[BC];
#pragma unroll
        for (int t = 0; t < BC; ++t) gv[t] = sG[t * LK + tid];
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < BC; ++t) {
            acc += gv[t];
            sG[t * LK + tid] = acc;
        }
    }
    __syncthreads();
    // wavefronts w and w + 4 share block row w: each forms two of its four blocks (j = 2 hv, 2 hv + 1)
    const int wi = tid >> 6, w = wi & 3, hv = wi >> 2, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    // A (strictly lower, beta applied) and P (lower with the diagonal, scale applied), block row w, with the
    // reference token b = 16 w: exp(G_t - G_s) = exp(G_t - G_b) exp(G_b - G_s). For the blocks left of the
    // diagonal (s < b <= t) both factors are at most 1. For the diagonal block (b <= s, t) the second factor is
    // at least 1; it is used when the block's decay range G_b - G_{b+15} is at most 64 on every channel (the
    // factor then stays below e^64), else the diagonal block takes the pairwise per-channel decays as they stand.
    {
        const int b0 = 16 * w;
        const float* Gb = sG + b0 * LK;
        bool wide = false;
        for (int c = lane; c < KD; c += 64) wide |= Gb[c] - sG[(b0 + 15) * LK + c] > 64.f;
        const bool fast = __ballot(wide) == 0;  // the same on every lane of the wavefront
        // All four blocks (w, j) as float32 MFMA tiles, without branches (the blocks right of the diagonal, and
        // the diagonal one when its range is wide, are formed and dropped; the exponent is clamped at 80 so that
        // they stay finite). Lane (ln, lg) brings A(t = b + ln, c) and B(c, s = 16 j + ln), c = kk + lg; four
        // reduction steps per pass, their reads issued together.
        f32x4 accA[2] = {zero4(), zero4()}, accP[2] = {zero4(), zero4()};
        const float* Kt = sK + (b0 + ln) * LK;
        const float* Qt = sQ + (b0 + ln) * LK;
        const float* Gt = sG + (b0 + ln) * LK;
        if constexpr (sizeof(ST) == 2) {
            // bf16 input: the decayed factors rounded to bf16, 32 channels per v_mfma_f32_16x16x32_bf16 (lane
            // (ln, lg) brings channels k0 + 8 lg .. + 7)
            typedef float f32x8 __attribute__((ext_vector_type(8)));
            for (int k0 = 0; k0 < KD; k0 += 32) {
                const int c0 = k0 + 8 * lg;
                f32x8 gb, ak, aq, gt, ks[2], gs[2];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const f32x4 g4 = *(const f32x4*)(Gb + c0 + 4 * hf), k4 = *(const f32x4*)(Kt + c0 + 4 * hf),
                                q4 = *(const f32x4*)(Qt + c0 + 4 * hf), t4 = *(const f32x4*)(Gt + c0 + 4 * hf);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        gb[4 * hf + e] = g4[e];
                        ak[4 * hf + e] = k4[e];
                        aq[4 * hf + e] = q4[e];
                        gt[4 * hf + e] = t4[e];
                    }
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj) {
                        const int j = 2 * hv + jj;
                        const f32x4 kk4 = *(const f32x4*)(sK + (16 * j + ln) * LK + c0 + 4 * hf),
                                    gg4 = *(const f32x4*)(sG + (16 * j + ln) * LK + c0 + 4 * hf);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            ks[jj][4 * hf + e] = kk4[e];
                            gs[jj][4 * hf + e] = gg4[e];
                        }
                    }
                }
                f32x8 a1, a2;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ft = __expf(gt[e] - gb[e]);
                    a1[e] = ak[e] * ft;
                    a2[e] = aq[e] * ft;
                }
                const bf16x8 A1 = __builtin_convertvector(a1, bf16x8), A2 = __builtin_convertvector(a2, bf16x8);
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    f32x8 bs;
#pragma unroll
                    for (int e = 0; e < 8; ++e) bs[e] = ks[jj][e] * __expf(fminf(gb[e] - gs[jj][e], 80.f));
                    const bf16x8 Bs = __builtin_convertvector(bs, bf16x8);
                    accA[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, Bs, accA[jj], 0, 0, 0);
                    accP[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A2, Bs, accP[jj], 0, 0, 0);
                }
            }
        } else
        for (int k0 = 0; k0 < KD; k0 += 16) {
            float gb[4], ak[4], aq[4], gt[4], ks[2][4], gs[2][4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = k0 + 4 * u + lg;
                gb[u] = Gb[c];
                ak[u] = Kt[c];
                aq[u] = Qt[c];
                gt[u] = Gt[c];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    ks[jj][u] = sK[(16 * (2 * hv + jj) + ln) * LK + c];
                    gs[jj][u] = sG[(16 * (2 * hv + jj) + ln) * LK + c];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float ft = __expf(gt[u] - gb[u]);
                const float a1 = ak[u] * ft, a2 = aq[u] * ft;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const float bs = ks[jj][u] * __expf(fminf(gb[u] - gs[jj][u], 80.f));
                    accA[jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, bs, accA[jj], 0, 0, 0);
                    accP[jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, bs, accP[jj], 0, 0, 0);
                }
            }
        }
        // the diagonal block with the pairwise decays: lane (ln = s, lg) forms rows t = b + 4 lg + r, four
        // channels at a time
        f32x4 da = zero4(), dp = zero4();
        if (!fast && hv == (w >> 1)) {  // (the wavefront holding the diagonal block)
            const int sd = b0 + ln;
#pragma unroll 2
            for (int c = 0; c < KD; c += 4) {
                const f32x4 ks = *(const f32x4*)(sK + sd * LK + c), gs = *(const f32x4*)(sG + sd * LK + c);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = b0 + 4 * lg + r;
                    const f32x4 kt = *(const f32x4*)(sK + t * LK + c), qt = *(const f32x4*)(sQ + t * LK + c),
                                gt = *(const f32x4*)(sG + t * LK + c);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // (clamped: only s <= t is kept, where G_t - G_s <= 0)
                        const float d = __expf(fminf(gt[e] - gs[e], 0.f)) * ks[e];
                        da[r] += kt[e] * d;
                        dp[r] += qt[e] * d;
                    }
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 2 * hv + jj, t = b0 + 4 * lg + r, s2 = 16 * j + ln;
                float a = 0.f, pv = 0.f;
                if (j < w) {
                    a = accA[jj][r];
                    pv = accP[jj][r];
                } else if (j == w) {
                    a = s2 < t ? (fast ? accA[jj][r] : da[r]) : 0.f;
                    pv = s2 <= t ? (fast ? accP[jj][r] : dp[r]) : 0.f;
                }
                sA[t * LL + s2] = sB[t] * a;
                sP[t * LL + s2] = scale * pv;
                sT[t * LL + s2] = 0.f;
            }
    }
    __syncthreads();
    constexpr bool B16 = sizeof(ST) == 2;
    typedef KdaRec16<KD> R16;
    float* R = rec + ((size_t)slot * H + h) * RL::floats(VD);
    uint8_t* const Rb = reinterpret_cast<uint8_t*>(R);  // the bf16 record's bytes
    static_assert(KdaRec16<KD>::bytes(VD) <= (3 * BC * KD + BC * VD + BC * BC + KD) * sizeof(float),
                  "the bf16 record fits in the float32 record's footprint");
    if (wi == 0) {
        // T: the four diagonal blocks at once, lane 16 bb + j solving column j of block bb: x_j = 1,
        // x_i = -sum_{j<=s<i} A_bb[i][s] x_s
        // (the column in registers; x_s = 0 for s < j, so the sums may start at 0)
        const int o = 16 * (lane >> 4), j = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = i == j ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < i; ++s2) acc -= sA[(o + i) * LL + o + s2] * x[s2];
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(o + i) * LL + o + j] = x[i];
    } else {
        // wavefronts 1-7: Qg = scale Gamma o Q and Kh = exp(G_L - G) o K to the record, K scaled by beta Gamma
        // in place (for W), Gamma_L and P to the record
        const int i0 = tid - 64, NS = NTP - 64;
        if constexpr (B16) {
            // (Kh^T and the scaled K follow once the solve no longer holds the wavefronts apart)
#pragma unroll 4
            for (int i = i0; i < BC * KD; i += NS) {
                const int tt = i / KD, c = i % KD;
                reinterpret_cast<bf16_t*>(Rb + R16::Q_OFF)[i] = f2bf(scale * __expf(sG[tt * LK + c]) * sQ[tt * LK + c]);
            }
            if (i0 < KD) reinterpret_cast<float*>(Rb + R16::gl_off(VD))[i0] = __expf(sG[(BC - 1) * LK + i0]);
            for (int i = i0; i < BC * BC; i += NS)
                reinterpret_cast<bf16_t*>(Rb + R16::P_OFF)[i] = f2bf(sP[(i / BC) * LL + i % BC]);
        } else {
#pragma unroll 4
            for (int i = i0; i < BC * KD; i += NS) {
                const int tt = i / KD, c = i % KD;
                const float G = sG[tt * LK + c], GL = sG[(BC - 1) * LK + c], kv = sK[tt * LK + c];
                const float eg = __expf(G);
                R[RL::q_off(VD) + i] = scale * eg * sQ[tt * LK + c];
                R[RL::kh_off(VD) + i] = __expf(GL - G) * kv;
                sK[tt * LK + c] = sB[tt] * eg * kv;
            }
            if (i0 < KD) R[RL::gl_off(VD) + i0] = __expf(sG[(BC - 1) * LK + i0]);
            for (int i = i0; i < BC * BC; i += NS) R[RL::p_off(VD) + i] = sP[(i / BC) * LL + i % BC];
        }
    }
    __syncthreads();
    tv.template store_rows<LK>(sV);  // (visible after the first barrier below)
    // T: off-diagonal blocks, one block diagonal dd at a time, block (i, j = i - dd) by wavefront i < 4
    for (int dd = 1; dd < 4; ++dd) {
        const int i = w, j = w - dd;
        if (hv == 0 && j >= 0) {
            // Ub = sum_{kb=j}^{i-1} A_i,kb T_kb,j (16 x 16, k over the tokens of blocks j .. i-1)
            const f32x4 Uv = mm4(sA + 16 * i * LL + 16 * j, LL, 1, sT + 16 * j * LL + 16 * j, LL, 1, 0, 16 * (i - j), zero4());
            float* Ub = sU + w * 16 * LU;
#pragma unroll
            for (int r = 0; r < 4; ++r) Ub[(4 * lg + r) * LU + ln] = Uv[r];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wavefront's own Ub tile is in LDS
            const f32x4 Tv = mm4(sT + 16 * i * LL + 16 * i, LL, 1, Ub, LU, 1, 0, 16, zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * lg + r) * LL + 16 * j + ln] = -Tv[r];
        }
        __syncthreads();
    }
    // V rows scaled by beta
    for (int i = tid; i < BC * VD; i += NTP) sV[(i / VD) * LK + i % VD] *= sB[i / VD];
    if constexpr (B16) {
        // Kh^T = (exp(G_L - G) o K)^T, consecutive threads along the tokens of one channel (contiguous stores)
#pragma unroll 4
        for (int i = tid; i < BC * KD; i += NTP) {
            const int c = i / BC, tt = i % BC;
            reinterpret_cast<bf16_t*>(Rb + R16::KT_OFF)[i] =
                f2bf(__expf(sG[(BC - 1) * LK + c] - sG[tt * LK + c]) * sK[tt * LK + c]);
        }
        __syncthreads();
        // K scaled by beta Gamma in place, for W
#pragma unroll 4
        for (int i = tid; i < BC * KD; i += NTP) {
            const int tt = i / KD, c = i % KD;
            sK[tt * LK + c] *= sB[tt] * __expf(sG[tt * LK + c]);
        }
    }
    __syncthreads();
    // W = T (beta Gamma o K), U = T (beta V): wavefront wi forms column tiles wi, wi + 8, .. of every row tile (T
    // is zero past column 16 ti + 15 of row tile ti), so the wavefronts share the triangle evenly
#pragma unroll
    for (int jc = wi; jc < NJ; jc += 8)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const f32x4 Wv = f32t::mmx<ST>(sT + 16 * ti * LL, LL, 1, sK + 16 * jc, LK, 1, 0, 16 * (ti + 1), zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (16 * ti + 4 * lg + r) * KD + 16 * jc + ln;
                if constexpr (B16)
                    reinterpret_cast<bf16_t*>(Rb + R16::W_OFF)[o] = f2bf(Wv[r]);
                else
                    R[RL::w_off() + o] = Wv[r];
            }
        }
#pragma unroll
    for (int jc = wi; jc < NV; jc += 8)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            const f32x4 Uv = f32t::mmx<ST>(sT + 16 * ti * LL, LL, 1, sV + 16 * jc, LK, 1, 0, 16 * (ti + 1), zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (16 * ti + 4 * lg + r) * VD + 16 * jc + ln;
                if constexpr (B16)
                    reinterpret_cast<float*>(Rb + R16::U_OFF)[o] = Uv[r];
                else
                    R[RL::u_off() + o] = Uv[r];
            }
        }
}

// ---------------------------------------------------------------------------------------------------------
// Chain: one 16-row slice of the state of one (sequence, head) through its chunks, on float32 MFMA tiles; the
// next chunk's record tiles load (into registers) while the current one computes. Wavefront w forms token tile w
// of R = U - W S^T, of Qg S^T and of O = Qg S^T + P R, and holds key tiles JPW w .. JPW w + JPW - 1 of the
// slice's state S [16][KD] (lane: rows 4 lg + r, key 16 jc + ln) for S <- S diag(Gamma_L) + R^T Kh; the state
// goes to LDS after each update as the B operand of the next chunk's products.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD, int VD>
__global__ __launch_bounds__(NT) void kda_chain_kernel(const float* __restrict__ h0, const int32_t* __restrict__ cu,
                                                       const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                       int T, int H, int n_seq, int nc, int nvs, ST* __restrict__ out,
                                                       float* __restrict__ ht) {
    typedef KdaRec<KD> RL;
    constexpr int LK = KD + 4, LL = BC + 1, LV = 17, JPW = KD / 64;
    __shared__ __align__(16) float sW[BC * LK];
    __shared__ __align__(16) float sQg[BC * LK];
    __shared__ __align__(16) float sKh[BC * LK];
    __shared__ __align__(16) float sS[16 * LK];
    __shared__ float sP[BC * LL], sU[BC * LV], sR[BC * LV], sGL[KD];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    int b, bos, eos, slot0;
    if (cu) {
        b = 0;
        bos = cu[n];
        eos = cu[n + 1];
        slot0 = chunk_off[n];
    } else {
        b = n;
        bos = 0;
        eos = T;
        slot0 = n * nc;
    }
    const int nch = (eos - bos + BC - 1) / BC;
    // the wavefront's key tiles of the state, C-tile layout
    f32x4 S[JPW];
#pragma unroll
    for (int i = 0; i < JPW; ++i) {
        const int c = 16 * (JPW * w + i) + ln;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[i][r] = h0 ? h0[(((size_t)n * H + h) * VD + v0 + 4 * lg + r) * KD + c] : 0.f;
    }
    Tile<float, BC, KD> tw, tq, tk;
    Tile<float, BC, BC> tp;
    Tile<float, BC, 16> tu;
    float gl = 0.f;
    auto recp = [&](int ci) __attribute__((always_inline)) { return rec + ((size_t)(slot0 + ci) * H + h) * RL::floats(VD); };
    // the next chunk's loads are issued in three groups spread over the step, each ahead of a stretch of
    // products, so that their issue (throttled by the memory pipeline) overlaps the computation
    auto issue_w = [&](int ci) __attribute__((always_inline)) {
        const float* R = recp(ci);
        tw.load(R + RL::w_off(), KD, BC);
        tu.load(R + RL::u_off() + v0, VD, BC);
        gl = tid < KD ? R[RL::gl_off(VD) + tid] : 0.f;
    };
    auto issue_q = [&](int ci) __attribute__((always_inline)) {
        const float* R = recp(ci);
        tq.load(R + RL::q_off(VD), KD, BC);
        tp.load(R + RL::p_off(VD), BC, BC);
    };
    auto issue_k = [&](int ci) __attribute__((always_inline)) { tk.load(recp(ci) + RL::kh_off(VD), KD, BC); };
    if (nch > 0) {
        issue_w(0);
        issue_q(0);
        issue_k(0);
    }
    const int tr0 = 16 * w + 4 * lg;
    for (int ci = 0; ci < nch; ++ci) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
#pragma unroll
        for (int i = 0; i < JPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sS[(4 * lg + r) * LK + 16 * (JPW * w + i) + ln] = S[i][r];
        tw.template store_rows<LK>(sW);
        tq.template store_rows<LK>(sQg);
        tk.template store_rows<LK>(sKh);
        tp.store(sP);
        tu.store(sU);
        if (tid < KD) sGL[tid] = gl;
        __syncthreads();
        const bool more = ci + 1 < nch;
        if (more) issue_w(ci + 1);
        // token tile w: R = U - W S^T and QS = Qg S^T (B(c, v) = S[v][c])
        const f32x4 WS = mm4(sW + 16 * w * LK, LK, 1, sS, 1, LK, 0, KD, zero4());
        if (more) issue_q(ci + 1);
        const f32x4 QS = mm4(sQg + 16 * w * LK, LK, 1, sS, 1, LK, 0, KD, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) sR[(tr0 + r) * LV + ln] = sU[(tr0 + r) * LV + ln] - WS[r];
        __syncthreads();
        if (more) issue_k(ci + 1);
        // O = QS + P R on token tile w (P is zero past column 16 w + 15)
        const f32x4 o = mm4(sP + 16 * w * LL, LL, 1, sR, LV, 1, 0, 16 * (w + 1), QS);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (tr0 + r < L) out[((row0 + tr0 + r) * H + h) * (long)VD + v0 + ln] = Elem<ST>::from_f(o[r]);
        // S <- S diag(Gamma_L) + R^T Kh on the wavefront's key tiles: A(v, t) = R[t][v], B(t, c) = Kh[t][c]
#pragma unroll
        for (int i = 0; i < JPW; ++i) {
            const int jc = JPW * w + i;
            S[i] = mm4(sR, 1, LV, sKh + 16 * jc, LK, 1, 0, BC, S[i] * sGL[16 * jc + ln]);
        }
        __syncthreads();
    }
    if (ht) {
#pragma unroll
        for (int i = 0; i < JPW; ++i) {
            const int c = 16 * (JPW * w + i) + ln;
#pragma unroll
            for (int r = 0; r < 4; ++r) ht[(((size_t)n * H + h) * VD + v0 + 4 * lg + r) * KD + c] = S[i][r];
        }
    }
}

// ---------------------------------------------------------------------------------------------------------
// Chain for bf16 input: the same steps as kda_chain_kernel with bf16 operands and float32 accumulation, from the
// bf16 record. The slice's state stays float32 in C-tile layout (rows v, key columns); its bf16 copy S_b [16][KD]
// and R^T in bf16 [16][64] go through LDS as the operands (every operand read is a 16-byte row read: W, Qg and P
// by token rows, S_b and R^T by value rows, Kh^T by key rows).
// ---------------------------------------------------------------------------------------------------------
template <int KD, int VD>
__global__ __launch_bounds__(NTP) void kda_chain16_kernel(const float* __restrict__ h0, const int32_t* __restrict__ cu,
                                                         const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                         int T, int H, int n_seq, int nc, int nvs, bf16_t* __restrict__ out,
                                                         float* __restrict__ ht) {
    typedef KdaRec<KD> RL;
    typedef KdaRec16<KD> R16;
    constexpr int LW = KD + 8, LT = BC + 8, LV = 17, JPW = KD / 64;
    __shared__ __align__(16) bf16_t sW[BC * LW];
    __shared__ __align__(16) bf16_t sQg[BC * LW];
    __shared__ __align__(16) bf16_t sKt[KD * LT];
    __shared__ __align__(16) bf16_t sP[BC * LT];
    __shared__ __align__(16) bf16_t sSb[16 * LW];
    __shared__ __align__(16) bf16_t sRt[16 * LT];
    __shared__ float sU[BC * LV], sGL[KD];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
    // wavefront wi: token tile w, half hv (half 0 forms R, half 1 Qg S^T and the output of the tile); key tile
    // JPW w + hv of the state (for K = 64 the wavefronts of half 1 hold none)
    const int wi = tid >> 6, w = wi & 3, hv = wi >> 2, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const bool own = hv < JPW;
    const int jc = JPW * w + hv;
    int b, bos, eos, slot0;
    if (cu) {
        b = 0;
        bos = cu[n];
        eos = cu[n + 1];
        slot0 = chunk_off[n];
    } else {
        b = n;
        bos = 0;
        eos = T;
        slot0 = n * nc;
    }
    const int nch = (eos - bos + BC - 1) / BC;
    f32x4 S = zero4();
    if (own && h0)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[r] = h0[(((size_t)n * H + h) * VD + v0 + 4 * lg + r) * KD + 16 * jc + ln];
    // a chunk's record tiles in registers (two sets: a chunk's loads are issued two steps before its step, in
    // three groups spread over the step, and the loop takes two steps per pass so that each set has fixed
    // registers)
    struct Ops16 {
        Tile<bf16_t, BC, KD, NTP> tw, tq;
        Tile<bf16_t, KD, BC, NTP> tk;
        Tile<bf16_t, BC, BC, NTP> tp;
        Tile<float, BC, 16, NTP> tu;
        float gl;
    } opA, opB;
    auto recb = [&](int ci) __attribute__((always_inline)) {
        return reinterpret_cast<const uint8_t*>(rec + ((size_t)(slot0 + ci) * H + h) * RL::floats(VD));
    };
    auto issue_w = [&](int ci, Ops16& o) __attribute__((always_inline)) {
        const uint8_t* R = recb(ci);
        o.tw.load(reinterpret_cast<const bf16_t*>(R + R16::W_OFF), KD, BC);
        o.tu.load(reinterpret_cast<const float*>(R + R16::U_OFF) + v0, VD, BC);
        o.gl = tid < KD ? reinterpret_cast<const float*>(R + R16::gl_off(VD))[tid] : 0.f;
    };
    auto issue_q = [&](int ci, Ops16& o) __attribute__((always_inline)) {
        const uint8_t* R = recb(ci);
        o.tq.load(reinterpret_cast<const bf16_t*>(R + R16::Q_OFF), KD, BC);
        o.tp.load(reinterpret_cast<const bf16_t*>(R + R16::P_OFF), BC, BC);
    };
    auto issue_k = [&](int ci, Ops16& o) __attribute__((always_inline)) {
        o.tk.load(reinterpret_cast<const bf16_t*>(recb(ci) + R16::KT_OFF), BC, KD);
    };
    const int tr0 = 16 * w + 4 * lg;
    auto step = [&](int ci, Ops16& o) __attribute__((always_inline)) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
        if (own)
#pragma unroll
            for (int r = 0; r < 4; ++r) sSb[(4 * lg + r) * LW + 16 * jc + ln] = f2bf(S[r]);
        o.tw.template store_raw<LW>(sW);
        o.tq.template store_raw<LW>(sQg);
        o.tk.template store_raw<LT>(sKt);
        o.tp.template store_raw<LT>(sP);
        o.tu.store(sU);
        if (tid < KD) sGL[tid] = o.gl;
        __syncthreads();
        const bool more = ci + 2 < nch;
        if (more) issue_w(ci + 2, o);
        // token tile w: R = U - W S^T (half 0) and QS = Qg S^T (half 1)
        if (more) issue_q(ci + 2, o);
        f32x4 QS = zero4();
        if (hv == 0) {
            const f32x4 WS = f32t::mmb(sW + 16 * w * LW, LW, sSb, LW, 0, KD, zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) sRt[ln * LT + tr0 + r] = f2bf(sU[(tr0 + r) * LV + ln] - WS[r]);
        } else {
            QS = f32t::mmb(sQg + 16 * w * LW, LW, sSb, LW, 0, KD, zero4());
        }
        __syncthreads();
        if (more) issue_k(ci + 2, o);
        // O = QS + P R on token tile w (P is zero past column 16 w + 15), by half 1
        if (hv == 1) {
            const f32x4 ov = f32t::mmb(sP + 16 * w * LT, LT, sRt, LT, 0, 16 * (w + 1), QS);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (tr0 + r < L) out[((row0 + tr0 + r) * H + h) * (long)VD + v0 + ln] = f2bf(ov[r]);
        }
        // S <- S diag(Gamma_L) + R^T Kh on the wavefront's key tile: A(v, t) = R^T[v][t], B(t, c) = Kh^T[c][t]
        if (own) S = f32t::mmb(sRt, LT, sKt + 16 * jc * LT, LT, 0, BC, S * sGL[16 * jc + ln]);
        __syncthreads();
    };
#pragma unroll
    for (int c = 0; c < 2; ++c)
        if (c < nch) {
            Ops16& o = c == 0 ? opA : opB;
            issue_w(c, o);
            issue_q(c, o);
            issue_k(c, o);
        }
    for (int ci = 0; ci < nch; ci += 2) {
        step(ci, opA);
        if (ci + 1 < nch) step(ci + 1, opB);
    }
    if (own && ht)
#pragma unroll
        for (int r = 0; r < 4; ++r) ht[(((size_t)n * H + h) * VD + v0 + 4 * lg + r) * KD + 16 * jc + ln] = S[r];
}

template <typename ST, int KD, int VD>
hipError_t run_kda(const ST* q, const ST* k, const ST* v, const float* g, const float* beta, const float* h0,
                   const int32_t* cu, const KdaWorkspace& ws, int N, int B, int T, int H, float scale, ST* out,
                   float* ht, hipStream_t s) {
    const bool packed = cu != nullptr;
    const long slots = gdn_slots(B, T, N, packed);
    const int nc = (T + BC - 1) / BC;
    hipError_t err;
    if (packed) {
        err = launch_chunk_table(cu, N, BC, slots, ws.chunk_off, ws.table, s);
        if (err != hipSuccess) return err;
    }
    if (slots > 0) {
        timing_begin("kda_prep", s);
        kda_prep_kernel<ST, KD, VD><<<dim3((unsigned)slots, H), NTP, 0, s>>>(q, k, v, g, beta, packed ? ws.table : nullptr,
                                                                           cu, T, H, nc, scale, ws.rec);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const long chains = (long)N * H;
    if (chains == 0) return hipSuccess;
    const int nvs = VD / 16;
    const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvs);
    timing_begin("kda_chain", s);
    if constexpr (sizeof(ST) == 2)
        kda_chain16_kernel<KD, VD><<<grid, NTP, 0, s>>>(h0, cu, ws.chunk_off, ws.rec, T, H, N, nc, nvs, out, ht);
    else
        kda_chain_kernel<ST, KD, VD><<<grid, NT, 0, s>>>(h0, cu, ws.chunk_off, ws.rec, T, H, N, nc, nvs, out, ht);
    timing_end(s);
    return hipGetLastError();
}

}  // namespace

size_t kda_record_floats(int K, int V) {
    return K == 128 ? KdaRec<128>::floats(V) : KdaRec<64>::floats(V);
}

hipError_t launch_kda_chunk(bool bf16, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* h0, const int32_t* cu, const KdaWorkspace& ws, int N,
                            int B, int T, int H, int K, int V, float scale, void* out, float* ht, hipStream_t s) {
#define SF_KDA_RUN(E, KK, VV)                                                                                      \
    return run_kda<E, KK, VV>(static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), g, beta, \
                              h0, cu, ws, N, B, T, H, scale, static_cast<E*>(out), ht, s)
    if (bf16) {
        if (K == 128 && V == 128) SF_KDA_RUN(bf16_t, 128, 128);
        if (K == 128 && V == 64) SF_KDA_RUN(bf16_t, 128, 64);
        SF_KDA_RUN(bf16_t, 64, 64);
    }
    if (K == 128 && V == 128) SF_KDA_RUN(float, 128, 128);
    if (K == 128 && V == 64) SF_KDA_RUN(float, 128, 64);
    SF_KDA_RUN(float, 64, 64);
#undef SF_KDA_RUN
}

}  // namespace sf

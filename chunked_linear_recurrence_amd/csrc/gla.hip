// Scalar-gated linear attention chunk forward for gfx950.
//
// S_t = exp(g_t) S_{t-1} + v_t k_t^T, o_t = scale S_t q_t (StateFlow Section
// 2.1, Eq. (1), with the scalar-identity transition of Mamba-2; the SSD core
// of the Megatron-LM page "Mamba2 state-passing context parallelism"). For
// one chunk of L <= C tokens with entry state S [V x K], cumulative gate G,
// Gamma_t = exp(G_t), e_t = exp(G_L - G_t), D_ti = exp(G_t - G_i) (i <= t):
//
//   O = scale (diag(Gamma) Q S^T + (D o Q K^T) V)
//   S <- Gamma_L S + (diag(e) V)^T K
//
// The state update does not depend on S beyond the scalar Gamma_L, so there
// is no solve and no separate Pre stage: each workgroup computes its chunk's
// masked Q K^T itself (the raw product is contracted first, then multiplied
// by decay differences of nonpositive exponent).
//
// Summary mode (Megatron-LM page: S_out = a_block S_in + S_ext): the state
// runs from zero without outputs; S_ext is its exit value and
// a_block = exp(sum of the gates).
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {

template <typename ST>
__device__ __forceinline__ ST gla_unit_elem(const u128& u, int e) {
    if constexpr (sizeof(ST) == 2) {
        const uint32_t w = u[e >> 1];
        return (ST)((e & 1) ? (w >> 16) : (w & 0xffffu));
    } else {
        return __uint_as_float(u[e]);
    }
}

template <typename ST, int KD, int C, int NW, bool SUMMARY>
__global__ __launch_bounds__(64 * NW) void gla_chain_kernel(
    const ST* __restrict__ q, const ST* __restrict__ k, const ST* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ h0, const int32_t* __restrict__ cu,
    int T, int H, int HK, int V, int n_seq, int nvb, float scale, ST* __restrict__ out,
    float* __restrict__ ht, float* __restrict__ a_out) {
    constexpr int E = 16 / sizeof(ST);
    constexpr int LDK = KD + E, LDC = C + E;
    constexpr int NT = 64 * NW;
    constexpr int KB = KD / 16;
    constexpr int CB = C / 16;
    constexpr int BV = 16 * NW;
    constexpr int UPR = KD / E;
    constexpr int NUK = C * UPR;
    constexpr int VPR = BV / E;            // units per token row of this block's V columns
    constexpr int NUV = C * VPR;
    constexpr int PK = (NUK + NT - 1) / NT;
    constexpr int PV = (NUV + NT - 1) / NT;
    constexpr int NPT = CB * (CB + 1) / 2;  // lower 16x16 tiles of the chunk
    constexpr int TPW = (NPT + NW - 1) / NW;
    // sK holds K while Q K^T is formed, then P (both C x (KD|C) with the larger ld)
    constexpr int LDKP = LDK > LDC ? LDK : LDC;
    constexpr int QSZ = SUMMARY ? E : C * LDK;
    typedef typename Elem<ST>::frag frag;

    __shared__ __align__(16) ST sKP[C * LDKP];
    __shared__ __align__(16) ST sKT[KD * LDC];
    __shared__ __align__(16) ST sQ[QSZ];
    __shared__ __align__(16) ST sVT[BV * LDC];
    __shared__ float sG[C], sGam[C], sE[C];
    __shared__ float sGL;

    int chain, vb;
    xcd_split(blockIdx.x, nvb, chain, vb);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, hk = h / (H / HK);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int v0 = vb * BV;
    const int myrow = v0 + 16 * wave + ln;

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
    const int nch = (eos - bos + C - 1) / C;

    f32x4 S[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int kk = 16 * kb + 4 * lg;
        if constexpr (!SUMMARY) {
            S[kb] = h0 ? *reinterpret_cast<const f32x4*>(h0 + (((size_t)n * H + h) * V + myrow) * KD + kk)
                       : zero4();
        } else {
            S[kb] = zero4();
        }
    }
    float gsum = 0.f;

    static_assert(NUK % NT == 0 && NUV % NT == 0, "staging units must divide evenly");
    // Unconditional loads from clamped rows; rows past the chunk end are
    // zeroed when the registers are written to LDS.
    u128 rk[PK], rq[PK], rv[PV];
    float rg;
    auto prefetch = [&](int c) __attribute__((always_inline)) {
        const int t0 = bos + c * C, L = min(C, eos - t0);
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int u = tid + i * NT;
            const int t = min(u / UPR, L - 1), col = (u % UPR) * E;
            const size_t off = ((size_t)(b * T + t0 + t) * HK + hk) * KD + col;
            rk[i] = *reinterpret_cast<const u128*>(k + off);
            if constexpr (!SUMMARY) rq[i] = *reinterpret_cast<const u128*>(q + off);
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int u = tid + i * NT;
            const int t = min(u / VPR, L - 1), col = (u % VPR) * E;
            rv[i] = *reinterpret_cast<const u128*>(v + ((size_t)(b * T + t0 + t) * H + h) * V + v0 + col);
        }
        rg = g[(size_t)(b * T + t0 + min(tid % C, L - 1)) * H + h];
    };

    if (nch > 0) prefetch(0);
    for (int c = 0; c < nch; ++c) {
        const int t0 = bos + c * C, L = min(C, eos - t0);
        const u128 zero = {0u, 0u, 0u, 0u};
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int u = tid + i * NT;
            const int t = u / UPR, col = (u % UPR) * E;
            const u128 kv = t < L ? rk[i] : zero;
            *reinterpret_cast<u128*>(sKP + t * LDKP + col) = kv;
#pragma unroll
            for (int e = 0; e < E; ++e) sKT[(col + e) * LDC + t] = gla_unit_elem<ST>(kv, e);
            if constexpr (!SUMMARY) *reinterpret_cast<u128*>(sQ + t * LDK + col) = t < L ? rq[i] : zero;
        }
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int u = tid + i * NT;
            const int t = u / VPR, col = (u % VPR) * E;
            const u128 vv = t < L ? rv[i] : zero;
#pragma unroll
            for (int e = 0; e < E; ++e) sVT[(col + e) * LDC + t] = gla_unit_elem<ST>(vv, e);
        }
        if (tid < C) sG[tid] = tid < L ? rg : 0.f;
        __syncthreads();
        if (c + 1 < nch) prefetch(c + 1);

        // within-chunk cumulative gate (wave 0), C / 64 tokens per lane
        if (wave == 0) {
            constexpr int PER = C / 64;
            float x[PER];
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                part += sG[PER * lane + j];
                x[j] = part;
            }
            const float incl = wave_inclusive_scan(part);
            const float base = incl - part;
#pragma unroll
            for (int j = 0; j < PER; ++j) x[j] += base;
            const float GL = __shfl(incl, 63, 64);
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const int t = PER * lane + j;
                sGam[t] = expf(x[j]);
                sE[t] = expf(GL - x[j]);
                sG[t] = x[j];
            }
            if (lane == 0) sGL = GL;
        }
        __syncthreads();
        gsum += sGL;

        if constexpr (!SUMMARY) {
            // P = scale (D o Q K^T) on the lower tiles, written over K
            f32x4 pt[TPW];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tt = wave + i * NW;
                pt[i] = zero4();
                if (tt < NPT) {
                    int ti = 0;
                    while ((ti + 1) * (ti + 2) / 2 <= tt) ++ti;
                    const int tj = tt - ti * (ti + 1) / 2;
                    f32x4 acc = zero4();
#pragma unroll
                    for (int kb = 0; kb < KB; kb += 2)
                        acc = Elem<ST>::mma2(acc, frag_rows(sQ, LDK, 16 * ti, 16 * kb), frag_rows(sQ, LDK, 16 * ti, 16 * kb + 16),
                                             frag_rows(sKP, LDKP, 16 * tj, 16 * kb), frag_rows(sKP, LDKP, 16 * tj, 16 * kb + 16));
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * ti + 4 * lg + r, j = 16 * tj + ln;
                        pt[i][r] = j <= t ? scale * expf(fminf(sG[t] - sG[j], 0.f)) * acc[r] : 0.f;
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tt = wave + i * NW;
                if (tt < NPT) {
                    int ti = 0;
                    while ((ti + 1) * (ti + 2) / 2 <= tt) ++ti;
                    const int tj = tt - ti * (ti + 1) / 2;
#pragma unroll
                    for (int r = 0; r < 4; ++r) sKP[(16 * ti + 4 * lg + r) * LDKP + 16 * tj + ln] = Elem<ST>::from_f(pt[i][r]);
                }
            }
            // the 32-token products below pair block (ti, ti) with the upper block (ti, ti+1) for even ti
            for (int ti = 2 * wave; ti < CB; ti += 2 * NW)
#pragma unroll
                for (int r = 0; r < 4; ++r) sKP[(16 * ti + 4 * lg + r) * LDKP + 16 * (ti + 1) + ln] = Elem<ST>::from_f(0.f);
            __syncthreads();

            frag Sb[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) Sb[kb] = Elem<ST>::pack(S[kb]);
#pragma unroll
            for (int ti = 0; ti < CB; ++ti) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; kb += 2)
                    acc = Elem<ST>::mma2(acc, frag_rows(sQ, LDK, 16 * ti, 16 * kb), frag_rows(sQ, LDK, 16 * ti, 16 * kb + 16),
                                         Sb[kb], Sb[kb + 1]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= scale * sGam[16 * ti + 4 * lg + r];
#pragma unroll
                for (int tj = 0; tj <= ti; tj += 2)
                    acc = Elem<ST>::mma2(acc, frag_rows(sKP, LDKP, 16 * ti, 16 * tj), frag_rows(sKP, LDKP, 16 * ti, 16 * tj + 16),
                                         frag_rows(sVT, LDC, 16 * wave, 16 * tj), frag_rows(sVT, LDC, 16 * wave, 16 * tj + 16));
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * ti + 4 * lg + r;
                    if (t < L) out[((size_t)(b * T + t0 + t) * H + h) * V + myrow] = Elem<ST>::from_f(acc[r]);
                }
            }
        }

        // S <- Gamma_L S + K^T (e V)
        frag EV[CB];
#pragma unroll
        for (int tb = 0; tb < CB; ++tb) {
            f32x4 x = Elem<ST>::unpack(frag_rows(sVT, LDC, 16 * wave, 16 * tb));
#pragma unroll
            for (int r = 0; r < 4; ++r) x[r] *= sE[16 * tb + 4 * lg + r];
            EV[tb] = Elem<ST>::pack(x);
        }
        const float gl = expf(sGL);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x4 acc = S[kb] * gl;
#pragma unroll
            for (int tb = 0; tb < CB; tb += 2)
                acc = Elem<ST>::mma2(acc, frag_rows(sKT, LDC, 16 * kb, 16 * tb), frag_rows(sKT, LDC, 16 * kb, 16 * tb + 16),
                                     EV[tb], EV[tb + 1]);
            S[kb] = acc;
        }
    }

#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int kk = 16 * kb + 4 * lg;
        if (ht) *reinterpret_cast<f32x4*>(ht + (((size_t)n * H + h) * V + myrow) * KD + kk) = S[kb];
    }
    if constexpr (SUMMARY) {
        if (vb == 0 && tid == 0) a_out[(size_t)n * H + h] = expf(gsum);
    }
}

template <typename ST, int KD, int C>
static hipError_t run_gla(int mode, const ST* q, const ST* k, const ST* v, const float* g,
                          const float* h0, const int32_t* cu, int N, int T, int H, int HK, int V,
                          float scale, ST* out, float* ht, float* a_out, hipStream_t s) {
    constexpr int NW = 4;
    const int nvb = V / (16 * NW);
    const int chains = N * H;
    if (chains == 0) return hipSuccess;
    const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvb);
    if (mode == 0) {
        timing_begin("gla_chain", s);
        gla_chain_kernel<ST, KD, C, NW, false><<<grid, 64 * NW, 0, s>>>(q, k, v, g, h0, cu, T, H, HK, V, N, nvb, scale, out, ht, nullptr);
    } else {
        timing_begin("gla_summary_chain", s);
        gla_chain_kernel<ST, KD, C, NW, true><<<grid, 64 * NW, 0, s>>>(q, k, v, g, nullptr, cu, T, H, HK, V, N, nvb, scale, nullptr, ht, a_out);
    }
    timing_end(s);
    return hipGetLastError();
}

template <typename ST>
static hipError_t gla_dispatch(int mode, const void* q, const void* k, const void* v, const float* g,
                               const float* h0, const int32_t* cu, int N, int T, int H, int HK, int K,
                               int V, int chunk, float scale, void* out, float* ht, float* a_out,
                               hipStream_t s) {
    const ST *qq = (const ST*)q, *kk = (const ST*)k, *vv = (const ST*)v;
    ST* oo = (ST*)out;
    if constexpr (sizeof(ST) == 2) {
        if (K == 128 && chunk == 128) return run_gla<ST, 128, 128>(mode, qq, kk, vv, g, h0, cu, N, T, H, HK, V, scale, oo, ht, a_out, s);
        if (K == 64 && chunk == 128) return run_gla<ST, 64, 128>(mode, qq, kk, vv, g, h0, cu, N, T, H, HK, V, scale, oo, ht, a_out, s);
    }
    if (chunk != 64) return hipErrorInvalidValue;  // float32 tiles of 128 tokens do not fit in LDS
    if (K == 128) return run_gla<ST, 128, 64>(mode, qq, kk, vv, g, h0, cu, N, T, H, HK, V, scale, oo, ht, a_out, s);
    return run_gla<ST, 64, 64>(mode, qq, kk, vv, g, h0, cu, N, T, H, HK, V, scale, oo, ht, a_out, s);
}

hipError_t launch_gla(bool bf16, int mode, const void* q, const void* k, const void* v,
                      const float* g, const float* h0, const int32_t* cu, int N, int B, int T,
                      int H, int HK, int K, int V, int chunk, float scale, void* out, float* ht,
                      float* a_out, hipStream_t s) {
    (void)B;
    if (bf16) return gla_dispatch<bf16_t>(mode, q, k, v, g, h0, cu, N, T, H, HK, K, V, chunk, scale, out, ht, a_out, s);
    return gla_dispatch<float>(mode, q, k, v, g, h0, cu, N, T, H, HK, K, V, chunk, scale, out, ht, a_out, s);
}

}  // namespace sf

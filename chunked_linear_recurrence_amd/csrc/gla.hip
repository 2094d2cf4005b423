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
#include <type_traits>

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

// ---------------------------------------------------------------------------
// bf16, V = 64: one workgroup of four wavefronts per (sequence, head) chain,
// two workgroups per CU (65.5 KB of LDS for K = 128, chunk 128).
//
// Per chunk, with K and V of the chunk in LDS (RowBlock layout, sf_device.h)
// and the bf16 entry state S_c in LDS:
//  - wavefront w forms, for its own token tiles (w and C/16-1-w for chunk 128,
//    w for chunk 64), P^T = scale (D o K Q^T)^T tile by tile from K rows in LDS
//    and its Q rows (registers, loaded during the previous chunk), and emits
//    O^T = scale diag(Gamma) (S_c Q^T) + V^T P^T for all 64 value rows;
//  - wavefront w updates the key columns it owns (KD/4 of them) of the float32
//    state, S <- Gamma_L S + (diag(e) V)^T K, from transposed reads of K and V.
// Then, after a barrier, the next chunk's K and V go straight into LDS with
// 16-byte direct loads, the gates are summed and the new bf16 state is
// written; a second barrier starts the next chunk. The other workgroup on the
// CU computes while one waits for its loads.
//
// Value rows inside a 16-row value tile vt follow the transposed V reads, which
// hand lane n the column v(vt, n) = 32 (vt / 2) + 8 (n / 4) + 4 (vt % 2) + n % 4;
// so lane group lg of an output tile holds the four consecutive rows
// 32 (vt / 2) + 8 lg + 4 (vt % 2) + r. State tiles: for key tile kt = 2p + h and
// value tile vt, lane (n, lg) holds S[v(vt, n)][32 p + 8 lg + 4 h + r], r = 0..3.
// ---------------------------------------------------------------------------
template <int KD, int C, bool SUMMARY>
__global__ __launch_bounds__(256, 2) void gla_bf16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ h0, const int32_t* __restrict__ cu,
    int T, int H, int HK, int n_seq, float scale, bf16_t* __restrict__ out, float* __restrict__ ht,
    float* __restrict__ a_out) {
    constexpr int V = 64, NVT = V / 16;
    constexpr int KP = KD / 32, KB = KD / 16, KTW = KB / 4;  // key tiles of the state per wavefront
    constexpr int NTT = C / 16;                              // token tiles per chunk
    constexpr int NOT = C == 128 ? 2 : 1;                    // output token tiles per wavefront
    typedef RowBlock<KD> RBk;
    typedef RowBlock<V> RBv;
    constexpr int UK = (16 / RBk::RPB) * 1024, UV = (16 / RBv::RPB) * 1024;  // bytes per 16 rows
    constexpr int OFF_K = 0;
    constexpr int OFF_V = OFF_K + C * RBk::RB;
    constexpr int OFF_SF = OFF_V + C * RBv::RB;          // [KB][NVT][64 lanes] x 8 B bf16 state
    constexpr int OFF_G = OFF_SF + KB * NVT * 512;       // G[C] (log2 units), Gamma[C], e[C], then G_L, Gamma_L
    constexpr int BYTES = OFF_G + 3 * C * 4 + 16;
    constexpr int NKI = C * RBk::RB / 1024 / 4, NVI = C * RBv::RB / 1024 / 4;  // direct loads per wavefront
    static_assert(NKI * 4 * 1024 == C * RBk::RB && NVI * 4 * 1024 == C * RBv::RB, "loads must divide evenly");
    static_assert(BYTES <= 80 * 1024, "two workgroups per CU");

    __shared__ __align__(16) uint8_t smem[BYTES];
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    typedef __attribute__((address_space(3))) float lds_f32;
    lds_u8* const lds0 = (lds_u8*)smem;
    lds_f32* const sG = (lds_f32*)(lds0 + OFF_G);
    lds_f32* const sGam = sG + C;
    lds_f32* const sE = sG + 2 * C;

    // the heads of one key group share K and Q rows: they run on one XCD
    const int GH = H / HK;
    int grp, j;
    xcd_split(blockIdx.x, GH, grp, j);
    if (grp >= n_seq * HK) return;
    const int n = grp / HK, hk = grp % HK, h = hk * GH + j;
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

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
    auto vrow = [&](int vt, int m) __attribute__((always_inline)) { return 32 * (vt >> 1) + 8 * (m >> 2) + 4 * (vt & 1) + (m & 3); };
    auto tile_of = [&](int i) __attribute__((always_inline)) { return i == 0 ? w : NTT - 1 - w; };

    // float32 state, own key tiles kt = w KTW + i
    f32x4 S[KTW][NVT];
#pragma unroll
    for (int i = 0; i < KTW; ++i)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            const int kt = w * KTW + i, kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1);
            S[i][vt] = (!SUMMARY && h0) ? *reinterpret_cast<const f32x4*>(h0 + (((size_t)n * H + h) * V + vrow(vt, ln)) * KD + kk)
                                        : zero4();
        }

    // ---- chunk c's K and V rows into LDS (rows past the end repeat the last token; their e = 0
    // keeps them out of the state and their outputs are not stored) and its gates into registers
    float rg[C / 64];
    // (the lane index is laundered through an empty asm so that the per-lane address terms are
    // formed here each time instead of being hoisted out of the chunk loop and kept live across it)
    auto load_chunk = [&](int c) __attribute__((always_inline)) {
        const int t0 = bos + c * C, L = min(C, eos - t0);
        int lo = lane;
        if constexpr (!SUMMARY) asm volatile("" : "+v"(lo));
#pragma unroll
        for (int i = 0; i < NKI; ++i) {
            const int m = w * NKI + i, r = m * RBk::RPB + lo / RBk::PCS;
            const int bb = (lo % RBk::PCS) ^ RBk::swz(r);
            load_lds16(k + ((size_t)(b * T + t0 + min(r, L - 1)) * HK + hk) * KD + 8 * bb, (uint8_t*)(lds0 + OFF_K + m * 1024));
        }
#pragma unroll
        for (int i = 0; i < NVI; ++i) {
            const int m = w * NVI + i, r = m * RBv::RPB + lo / RBv::PCS;
            const int bb = (lo % RBv::PCS) ^ RBv::swz(r);
            load_lds16(v + ((size_t)(b * T + t0 + min(r, L - 1)) * H + h) * V + 8 * bb, (uint8_t*)(lds0 + OFF_V + m * 1024));
        }
        if (w == 0) {
#pragma unroll
            for (int i = 0; i < C / 64; ++i) {
                const int t = (C / 64) * lo + i;
                rg[i] = t < L ? g[(size_t)(b * T + t0 + t) * H + h] : 0.f;
            }
        }
    };
    // cumulative gate of the chunk (wavefront 0, after its loads landed); padded gates are 0, so
    // the total is G at the last token
    auto gates = [&](int c) __attribute__((always_inline)) {
        const int t0 = bos + c * C, L = min(C, eos - t0);
        constexpr int PER = C / 64;
        float x[PER], part = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            part += rg[i];
            x[i] = part;
        }
        const float incl = wave_inclusive_scan(part), base = incl - part;
        const float GL = __shfl(incl, 63, 64);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int t = PER * lane + i;
            const float G = base + x[i];
            sG[t] = G * 1.4426950408889634f;  // log2 units: the decay masks use the hardware exp2
            sGam[t] = __expf(G);
            sE[t] = t < L ? __expf(GL - G) : 0.f;
        }
        if (lane == 0) {
            sG[3 * C] = GL;
            sG[3 * C + 1] = __expf(GL);
        }
    };
    auto store_state = [&]() __attribute__((always_inline)) {  // bf16 copy of own state tiles
        lds_u8* B = lds0 + OFF_SF + lane * 8;
#pragma unroll
        for (int i = 0; i < KTW; ++i)
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt)
                *(lds_i16x4*)(B + ((w * KTW + i) * NVT + vt) * 512) = Elem<bf16_t>::pack(S[i][vt]);
    };
    // Q rows of own output tiles: lane (ln, lg) <- Q[16 tt + ln][32 p + 8 lg + j]
    bf16x8 Q[NOT][KP];
    auto load_q = [&](int c) __attribute__((always_inline)) {
        const int t0 = bos + c * C, L = min(C, eos - t0);
        int lo = lane;
        asm volatile("" : "+v"(lo));
#pragma unroll
        for (int i = 0; i < NOT; ++i) {
            const bf16_t* qr = q + ((size_t)(b * T + t0 + min(16 * tile_of(i) + (lo & 15), L - 1)) * HK + hk) * KD + 8 * (lo >> 4);
#pragma unroll
            for (int p = 0; p < KP; ++p) Q[i][p] = *reinterpret_cast<const bf16x8*>(qr + 32 * p);
        }
    };
    auto prologue_sync = [&](int c) __attribute__((always_inline)) {  // loads of chunk c landed -> gates
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (w == 0) gates(c);
    };

    float gsum = 0.f;
    if (nch > 0) {
        load_chunk(0);
        if constexpr (!SUMMARY) {
            load_q(0);
            store_state();
        }
        prologue_sync(0);
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int t0 = bos + c * C, L = min(C, eos - t0);
        if constexpr (SUMMARY) gsum += sG[3 * C];
        // ---- compute phase, specialised per wavefront so that every tile bound is a constant
        auto compute = [&](auto WC) __attribute__((always_inline)) {
            constexpr int WV = decltype(WC)::value;
            // lane-dependent LDS offsets are formed here each chunk (laundered lane index) rather than
            // kept live across the chunk loop
            int lo = lane;
            if constexpr (!SUMMARY) asm volatile("" : "+v"(lo));
            const int ln = lo & 15, lg = lo >> 4;
            // key tiles depend on the wavefront only through kw; the summary pass has no output tiles
            // and keeps one body with the runtime index (four copies cost more than they save there)
            const int kw = SUMMARY ? w : WV;
            // ---- output tiles: P^T fragments of own token tiles
            bf16x8 Pf[NOT][NTT / 2];
            float gam[NOT];
            if constexpr (!SUMMARY) {
#pragma unroll
                for (int i = 0; i < NOT; ++i) {
                    const int tt = i == 0 ? WV : NTT - 1 - WV;
                    const float Gt = sG[16 * tt + ln];
                    gam[i] = sGam[16 * tt + ln] * scale;
                    f32x4 PT[NTT];
#pragma unroll
                    for (int si = 0; si < NTT; ++si) {
                        PT[si] = zero4();
                        if (si <= tt) {
#pragma unroll
                            for (int p = 0; p < KP; ++p)
                                PT[si] = mma32(*(lds_bf16x8*)(lds0 + OFF_K + RBk::off(ln, 4 * p + lg) + si * UK), Q[i][p], PT[si]);
                            const f32x4 Gs = *(lds_f32x4*)(sG + 16 * si + 4 * lg);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                // token s = 16 si + 4 lg + r against t = 16 tt + ln: only s <= t, where G_t - G_s <= 0
                                const bool keep = si < tt || 4 * lg + r <= ln;
                                PT[si][r] = keep ? PT[si][r] * (scale * __builtin_amdgcn_exp2f(fminf(Gt - Gs[r], 0.f))) : 0.f;
                            }
                        }
                    }
#pragma unroll
                    for (int pp = 0; pp < NTT / 2; ++pp) Pf[i][pp] = cat8(Elem<bf16_t>::pack(PT[2 * pp]), Elem<bf16_t>::pack(PT[2 * pp + 1]));
                }
            }
            // ---- own key tiles of K^T: lane (n, lg) <- K[16 u + 4 lg + r][32 p + 8 (n/4) + 4 h + n%4]
            i16x4 Ka[KTW][NTT];
#pragma unroll
            for (int i = 0; i < KTW; ++i) {
                const int kt = kw * KTW + i;
                const int ktr = RBk::off(4 * lg + (ln >> 2), 4 * (kt >> 1) + (ln & 3)) + 8 * (kt & 1);
#pragma unroll
                for (int u = 0; u < NTT; ++u) Ka[i][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds0 + OFF_K + ktr + u * UK));
            }
            // the update's factor e_t scales token t's key row here, once per chunk (the wavefront's
            // own key tiles only), rather than its value row in every value tile: sum_t (e_t k_t) v_t^T
            // is the same sum, and the output keeps the unscaled V
#pragma unroll
            for (int u = 0; u < NTT; ++u) {
                const f32x4 eu = *(lds_f32x4*)(sE + 16 * u + 4 * lg);
#pragma unroll
                for (int i = 0; i < KTW; ++i) Ka[i][u] = Elem<bf16_t>::pack(Elem<bf16_t>::unpack(Ka[i][u]) * eu);
            }
            const float gamL = sG[3 * C + 1];
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) {
                // V^T fragments of value tile vt: lane (n, lg) <- V[16 u + 4 lg + r][v(vt, n)]
                const int vtr = RBv::off(4 * lg + (ln >> 2), 4 * (vt >> 1) + (ln & 3)) + 8 * (vt & 1);
                i16x4 Vt[NTT];
#pragma unroll
                for (int u = 0; u < NTT; ++u) Vt[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds0 + OFF_V + vtr + u * UV));
                if constexpr (!SUMMARY) {
                    // bf16 entry state of value tile vt, all key columns (A operand: rows v, columns k)
                    bf16x8 Sq[KP];
                    lds_u8* sb = lds0 + OFF_SF + lane * 8 + vt * 512;
#pragma unroll
                    for (int p = 0; p < KP; ++p)
                        Sq[p] = cat8(*(lds_i16x4*)(sb + (2 * p) * NVT * 512), *(lds_i16x4*)(sb + (2 * p + 1) * NVT * 512));
#pragma unroll
                    for (int i = 0; i < NOT; ++i) {
                        const int tt = i == 0 ? WV : NTT - 1 - WV, t = 16 * tt + ln;
                        f32x4 o = zero4();
#pragma unroll
                        for (int p = 0; p < KP; ++p) o = mma32(Sq[p], Q[i][p], o);
                        o = o * gam[i];
#pragma unroll
                        for (int pp = 0; pp < NTT / 2; ++pp)
                            if (pp <= tt / 2) o = mma32(cat8(Vt[2 * pp], Vt[2 * pp + 1]), Pf[i][pp], o);
                        if (t < L)
                            *reinterpret_cast<i16x4*>(out + ((size_t)(b * T + t0 + t) * H + h) * V + vrow(vt, 4 * lg)) = Elem<bf16_t>::pack(o);
                    }
                }
                // S[:, own keys] of tile vt <- Gamma_L S + V^T (e K)
#pragma unroll
                for (int i = 0; i < KTW; ++i) {
                    f32x4 acc = S[i][vt] * gamL;
#pragma unroll
                    for (int uu = 0; uu < NTT / 2; ++uu) acc = mma32(cat8(Ka[i][2 * uu], Ka[i][2 * uu + 1]), cat8(Vt[2 * uu], Vt[2 * uu + 1]), acc);
                    S[i][vt] = acc;
                }
            }
        };
        if constexpr (SUMMARY) compute(std::integral_constant<int, 0>{});
        else switch (w) {
            case 0: compute(std::integral_constant<int, 0>{}); break;
            case 1: compute(std::integral_constant<int, 1>{}); break;
            case 2: compute(std::integral_constant<int, 2>{}); break;
            default: compute(std::integral_constant<int, 3>{}); break;
        }
        const bool more = c + 1 < nch;
        if constexpr (!SUMMARY)
            if (more) load_q(c + 1);  // lands during the exchange below
        __syncthreads();
        if (more) {
            load_chunk(c + 1);
            if constexpr (!SUMMARY) store_state();
            prologue_sync(c + 1);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < KTW; ++i)
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt) {
            const int kt = w * KTW + i, kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1);
            if (ht) *reinterpret_cast<f32x4*>(ht + (((size_t)n * H + h) * V + vrow(vt, ln)) * KD + kk) = S[i][vt];
        }
    if constexpr (SUMMARY) {
        if (tid == 0) a_out[(size_t)n * H + h] = expf(gsum);
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

template <int KD, int C>
static hipError_t run_gla_bf16(int mode, const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* g,
                               const float* h0, const int32_t* cu, int N, int T, int H, int HK, float scale,
                               bf16_t* out, float* ht, float* a_out, hipStream_t s) {
    const int groups = N * HK;
    if (groups == 0) return hipSuccess;
    const unsigned grid = (unsigned)(((groups + 7) / 8) * 8 * (H / HK));
    if (mode == 0) {
        timing_begin("gla_chain", s);
        gla_bf16_kernel<KD, C, false><<<grid, 256, 0, s>>>(q, k, v, g, h0, cu, T, H, HK, N, scale, out, ht, nullptr);
    } else {
        timing_begin("gla_summary_chain", s);
        gla_bf16_kernel<KD, C, true><<<grid, 256, 0, s>>>(q, k, v, g, nullptr, cu, T, H, HK, N, scale, nullptr, ht, a_out);
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
        if (V == 64 && (K == 128 || K == 64) && (chunk == 128 || chunk == 64)) {
            if (K == 128 && chunk == 128) return run_gla_bf16<128, 128>(mode, qq, kk, vv, g, h0, cu, N, T, H, HK, scale, oo, ht, a_out, s);
            if (K == 128) return run_gla_bf16<128, 64>(mode, qq, kk, vv, g, h0, cu, N, T, H, HK, scale, oo, ht, a_out, s);
            if (chunk == 128) return run_gla_bf16<64, 128>(mode, qq, kk, vv, g, h0, cu, N, T, H, HK, scale, oo, ht, a_out, s);
            return run_gla_bf16<64, 64>(mode, qq, kk, vv, g, h0, cu, N, T, H, HK, scale, oo, ht, a_out, s);
        }
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

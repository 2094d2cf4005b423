// Gated Delta Rule chunk forward for gfx950.
//
// The recurrence (attention-gym "Linear Attention", section "Gated Delta
// Rule") is run chunk by chunk with the Pre / ST / Out split of StateFlow
// (Section 2.2, Eq. (2)). For one chunk of L <= 64 tokens of one (sequence,
// value head), entry state S [V x K], within-chunk cumulative gate G,
// Gamma_t = exp(G_t), e_t = exp(G_L - G_t), D_ti = exp(G_t - G_i) (i <= t):
//
//   Pre (state independent, all chunks in parallel)   -> gdn_prep_kernel
//     A = diag(beta) (strictly-lower D o K K^T),  T = (I + A)^-1
//     P = scale (D o Q K^T)   (lower triangle incl. diagonal)
//   ST + Out (serial over chunks)                      -> gdn_chain_kernel
//     X = K S^T,  Y = diag(beta) (V - diag(Gamma) X),  R = T Y
//     O = scale diag(Gamma) Q S^T + P R
//     S <- Gamma_L S + (diag(e) R)^T K
//
// R is the chunk's corrected values (the residuals of the token rule). The
// masked products are contracted raw and then multiplied by decay factors
// exp(G_t - G_i) with i <= t only, so nothing overflows however negative the
// gates are (the gate has no lower bound). Every contraction is a 16x16 MFMA
// block product (sf_device.h); the state is carried in float32 and fed to
// the MFMA in the q/k/v element type, as the page allows for the chunk-entry
// state.
//
// Value rows of the state are independent, so one workgroup handles
// 16 * NW rows (one 16-row slice per wavefront) of one (sequence, head)
// chain, and the rows of a chain are spread over several workgroups placed
// on one XCD.
//
// Summary mode (attention-gym "Context Parallelism", "cuDNN local
// execution"): the chain runs on V + K rows, the first V from a zero state
// with the values, the last K from the identity with the values disabled;
// their exit states are S_ext and the transition M.
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {

constexpr int GC = kGdnChunk;

// ---------------------------------------------------------------------------
// Chunk table of packed inputs: chunk_off[n] = first chunk slot of sequence n
// (exclusive prefix of ceil(len_n / C)), table[s] = (sequence, chunk index)
// or (-1, 0) past the last chunk. One workgroup.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void chunk_table_kernel(const int32_t* __restrict__ cu, int N,
                                                          int C, int cap, int* __restrict__ chunk_off,
                                                          int2* __restrict__ table) {
    __shared__ int s_scan[256];
    __shared__ int s_run;
    const int tid = threadIdx.x;
    if (tid == 0) s_run = 0;
    __syncthreads();
    for (int base = 0; base < N; base += 256) {
        const int n = base + tid;
        int cnt = 0;
        if (n < N) cnt = (cu[n + 1] - cu[n] + C - 1) / C;
        s_scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int y = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += y;
            __syncthreads();
        }
        const int run = s_run;
        if (n < N) chunk_off[n] = run + s_scan[tid] - cnt;
        __syncthreads();
        if (tid == 255) s_run = run + s_scan[255];
        __syncthreads();
    }
    const int total = s_run;
    if (tid == 0) chunk_off[N] = total;
    __threadfence();
    __syncthreads();
    for (int s = tid; s < cap; s += 256) {
        int2 e = make_int2(-1, 0);
        if (s < total) {
            // last sequence whose first slot is <= s (empty sequences repeat offsets)
            int lo = 0, hi = N - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (chunk_off[mid] <= s) lo = mid; else hi = mid - 1;
            }
            e = make_int2(lo, s - chunk_off[lo]);
        }
        table[s] = e;
    }
}

// Locate chunk `slot`: batch row, first token, length. false past the end.
__device__ __forceinline__ bool chunk_coords(int slot, const int2* table, const int32_t* cu, int T,
                                             int nc, int& b, int& t0, int& L) {
    if (table) {
        const int2 e = table[slot];
        if (e.x < 0) return false;
        b = 0;
        t0 = cu[e.x] + GC * e.y;
        L = min(GC, cu[e.x + 1] - t0);
    } else {
        b = slot / nc;
        t0 = (slot % nc) * GC;
        L = min(GC, T - t0);
    }
    return true;
}

// ---------------------------------------------------------------------------
// Pre: per (chunk slot, head) -> T, P, coefficients.
// Record layout: T [64][64] ST | P [64][64] ST | coef float[256]:
//   [0,64) Gamma_t  [64,128) e_t  [128,192) beta_t  [192] Gamma_L
// ---------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(256) void gdn_prep_kernel(const ST* __restrict__ q, const ST* __restrict__ k,
                                                       const float* __restrict__ g,
                                                       const float* __restrict__ beta,
                                                       const int2* __restrict__ table,
                                                       const int32_t* __restrict__ cu, int T, int H,
                                                       int HK, int nc, float scale, int want_p,
                                                       uint8_t* __restrict__ fac) {
    constexpr int E = 16 / sizeof(ST);  // elements per 16-byte unit
    constexpr int LDK = KD + E, LD = GC + E;
    constexpr int UPR = KD / E;
    __shared__ __align__(16) ST sK[GC * LDK];
    __shared__ __align__(16) ST sQ[GC * LDK];
    __shared__ __align__(16) ST sP[GC * LD];
    __shared__ float sA[GC * 65];
    __shared__ float sT[GC * 65];
    __shared__ float sX[3 * 256];
    __shared__ float sG[GC], sB[GC];

    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const int hk = h / (H / HK);

    for (int u = tid; u < GC * UPR; u += 256) {
        const int t = u / UPR, c = (u % UPR) * E;
        u128 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
        if (t < L) {
            const size_t off = ((size_t)(b * T + t0 + t) * HK + hk) * KD + c;
            kv = *reinterpret_cast<const u128*>(k + off);
            if (want_p) qv = *reinterpret_cast<const u128*>(q + off);
        }
        *reinterpret_cast<u128*>(sK + t * LDK + c) = kv;
        *reinterpret_cast<u128*>(sQ + t * LDK + c) = qv;
    }
    if (tid < GC) {
        const size_t gi = (size_t)(b * T + t0 + tid) * H + h;
        const float gv = tid < L ? g[gi] : 0.f;
        sB[tid] = tid < L ? beta[gi] : 0.f;
        sG[tid] = wave_inclusive_scan(gv);
    }
    for (int i = tid; i < GC * 65; i += 256) sT[i] = 0.f;
    for (int i = tid; i < GC * LD; i += 256) sP[i] = Elem<ST>::from_f(0.f);
    __syncthreads();

    uint8_t* rec = fac + ((size_t)slot * H + h) * gdn_factor_bytes(sizeof(ST));
    ST* gT = reinterpret_cast<ST*>(rec);
    ST* gP = gT + GC * GC;
    float* gC = reinterpret_cast<float*>(gP + GC * GC);
    if (tid < GC) {
        const float G = sG[tid], GL = sG[GC - 1];
        gC[tid] = expf(G);
        gC[64 + tid] = expf(GL - G);
        gC[128 + tid] = sB[tid];
        gC[192 + tid] = tid == 0 ? expf(GL) : 0.f;
    }

    // raw K K^T and Q K^T on the 10 lower 16x16 tiles each, then decay masks
    const int wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int ntiles = want_p ? 20 : 10;
    for (int it = wave; it < ntiles; it += 4) {
        const bool isP = it >= 10;
        const int tt = isP ? it - 10 : it;
        const int ti = (tt >= 1) + (tt >= 3) + (tt >= 6);
        const int tj = tt - ti * (ti + 1) / 2;
        const ST* X = isP ? sQ : sK;
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KD / 16; ++kb)
            acc = Elem<ST>::mma(acc, frag_rows(X, LDK, 16 * ti, 16 * kb), frag_rows(sK, LDK, 16 * tj, 16 * kb));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * ti + 4 * lg + r, i = 16 * tj + ln;
            const float d = expf(fminf(sG[t] - sG[i], 0.f));
            if (isP) {
                sP[t * LD + i] = Elem<ST>::from_f(i <= t ? scale * d * acc[r] : 0.f);
            } else {
                sA[t * 65 + i] = i < t ? sB[t] * d * acc[r] : 0.f;
            }
        }
    }
    __syncthreads();

    // T = (I + A)^-1: the four 16x16 diagonal blocks by forward substitution
    // (one lane per column), then the off-diagonal blocks by block rows:
    // T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.
    if (wave == 0) {
        const int blk = lane >> 4, j = lane & 15;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float s = (t == j) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < t; ++i) s -= sA[(16 * blk + t) * 65 + 16 * blk + i] * x[i];
            x[t] = s;
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) sT[(16 * blk + t) * 65 + 16 * blk + j] = x[t];
    }
    __syncthreads();
    const int er = tid >> 4, ec = tid & 15;
    for (int d = 1; d < 4; ++d) {
        for (int i = d; i < 4; ++i) {
            const int j = i - d;
            float s = 0.f;
            for (int m = j; m < i; ++m)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    s += sA[(16 * i + er) * 65 + 16 * m + kk] * sT[(16 * m + kk) * 65 + 16 * j + ec];
            sX[(i - d) * 256 + tid] = s;
        }
        __syncthreads();
        for (int i = d; i < 4; ++i) {
            const int j = i - d;
            float s = 0.f;
            for (int kk = 0; kk <= er; ++kk)
                s += sT[(16 * i + er) * 65 + 16 * i + kk] * sX[(i - d) * 256 + kk * 16 + ec];
            sT[(16 * i + er) * 65 + 16 * j + ec] = -s;
        }
        __syncthreads();
    }

    for (int i = tid; i < GC * GC; i += 256) gT[i] = Elem<ST>::from_f(sT[(i >> 6) * 65 + (i & 63)]);
    if (want_p) {
        constexpr int UR = GC / E;
        for (int u = tid; u < GC * UR; u += 256) {
            const int r = u / UR, c = (u % UR) * E;
            *reinterpret_cast<u128*>(gP + r * GC + c) = *reinterpret_cast<const u128*>(sP + r * LD + c);
        }
    }
}

// ---------------------------------------------------------------------------
// ST + Out: one workgroup = NW wavefronts = 16*NW state rows of one chain.
// ---------------------------------------------------------------------------
template <typename ST>
__device__ __forceinline__ ST unit_elem(const u128& u, int e) {
    if constexpr (sizeof(ST) == 2) {
        const uint32_t w = (&u.x)[e >> 1];
        return (ST)((e & 1) ? (w >> 16) : (w & 0xffffu));
    } else {
        return __uint_as_float((&u.x)[e]);
    }
}

template <typename ST, int KD, int NW, bool SUMMARY>
__global__ __launch_bounds__(64 * NW) void gdn_chain_kernel(
    const ST* __restrict__ q, const ST* __restrict__ k, const ST* __restrict__ v,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const uint8_t* __restrict__ fac, int T, int H, int HK, int V, int n_seq, int nc, int nvb,
    float scale, ST* __restrict__ out, float* __restrict__ ht, float* __restrict__ Mout) {
    constexpr int E = 16 / sizeof(ST);
    constexpr int LDK = KD + E, LD = GC + E;
    constexpr int NT = 64 * NW;
    constexpr int KB = KD / 16;
    constexpr int UPR = KD / E;             // units per K/Q row
    constexpr int NUK = GC * UPR;           // units per K (or Q) chunk
    constexpr int NUT = GC * GC / E;        // units per T (or P) block
    constexpr int PK = (NUK + NT - 1) / NT;
    constexpr int PT = (NUT + NT - 1) / NT;
    constexpr int QSZ = SUMMARY ? E : GC * LDK;
    constexpr int PSZ = SUMMARY ? E : GC * LD;
    typedef typename Elem<ST>::frag frag;

    __shared__ __align__(16) ST sK[GC * LDK];
    __shared__ __align__(16) ST sKT[KD * LD];
    __shared__ __align__(16) ST sQ[QSZ];
    __shared__ __align__(16) ST sT[GC * LD];
    __shared__ __align__(16) ST sP[PSZ];
    __shared__ __align__(16) float sC[256];

    int chain, vb;
    xcd_split(blockIdx.x, nvb, chain, vb);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, hk = h / (H / HK);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int myrow = (vb * NW + wave) * 16 + ln;
    const bool vrow = myrow < V;

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
    const int nch = (eos - bos + GC - 1) / GC;
    const size_t rec_bytes = gdn_factor_bytes(sizeof(ST));

    // state S^T as KB C tiles: lane holds S[myrow][16 kb + 4 lg + r]
    f32x4 S[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int kk = 16 * kb + 4 * lg;
        if constexpr (!SUMMARY) {
            S[kb] = h0 ? *reinterpret_cast<const f32x4*>(h0 + (((size_t)n * H + h) * V + myrow) * KD + kk)
                       : zero4();
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) S[kb][r] = (!vrow && kk + r == myrow - V) ? 1.f : 0.f;
        }
    }

    u128 rk[PK], rq[PK], rt[PT], rp[PT], rc;
    ST rv[16];
    auto prefetch = [&](int c) {
        const int t0 = bos + c * GC, L = min(GC, eos - t0);
        const uint8_t* rec = fac + ((size_t)(slot0 + c) * H + h) * rec_bytes;
        const ST* gT = reinterpret_cast<const ST*>(rec);
        const ST* gP = gT + GC * GC;
        const float* gC = reinterpret_cast<const float*>(gP + GC * GC);
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int u = tid + i * NT;
            rk[i] = rq[i] = u128{0u, 0u, 0u, 0u};
            if (u < NUK) {
                const int t = u / UPR, col = (u % UPR) * E;
                if (t < L) {
                    const size_t off = ((size_t)(b * T + t0 + t) * HK + hk) * KD + col;
                    rk[i] = *reinterpret_cast<const u128*>(k + off);
                    if constexpr (!SUMMARY) rq[i] = *reinterpret_cast<const u128*>(q + off);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + i * NT;
            if (u < NUT) {
                rt[i] = *reinterpret_cast<const u128*>(gT + u * E);
                if constexpr (!SUMMARY) rp[i] = *reinterpret_cast<const u128*>(gP + u * E);
            }
        }
        if (tid < 64) rc = *reinterpret_cast<const u128*>(gC + 4 * tid);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * (i >> 2) + 4 * lg + (i & 3);
            rv[i] = (vrow && t < L) ? v[((size_t)(b * T + t0 + t) * H + h) * V + myrow] : Elem<ST>::from_f(0.f);
        }
    };

    if (nch > 0) prefetch(0);
    for (int c = 0; c < nch; ++c) {
        const int t0 = bos + c * GC, L = min(GC, eos - t0);
        __syncthreads();
        // registers -> LDS (K natural and transposed, Q, T, P, coefficients)
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int u = tid + i * NT;
            if (u < NUK) {
                const int t = u / UPR, col = (u % UPR) * E;
                *reinterpret_cast<u128*>(sK + t * LDK + col) = rk[i];
#pragma unroll
                for (int e = 0; e < E; ++e) sKT[(col + e) * LD + t] = unit_elem<ST>(rk[i], e);
                if constexpr (!SUMMARY) *reinterpret_cast<u128*>(sQ + t * LDK + col) = rq[i];
            }
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + i * NT;
            if (u < NUT) {
                const int r = u / (GC / E), col = (u % (GC / E)) * E;
                *reinterpret_cast<u128*>(sT + r * LD + col) = rt[i];
                if constexpr (!SUMMARY) *reinterpret_cast<u128*>(sP + r * LD + col) = rp[i];
            }
        }
        if (tid < 64) *reinterpret_cast<u128*>(sC + 4 * tid) = rc;
        float vv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) vv[i] = Elem<ST>::to_f(rv[i]);
        __syncthreads();
        if (c + 1 < nch) prefetch(c + 1);

        frag Sb[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Sb[kb] = Elem<ST>::pack(S[kb]);

        // X = K S^T ; Y = beta (V - Gamma X)
        frag Yb[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) acc = Elem<ST>::mma(acc, frag_rows(sK, LDK, 16 * tb, 16 * kb), Sb[kb]);
            f32x4 y;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tb + 4 * lg + r;
                y[r] = sC[128 + t] * (vv[4 * tb + r] - sC[t] * acc[r]);
            }
            Yb[tb] = Elem<ST>::pack(y);
        }
        // R = T Y
        f32x4 R[4];
        frag Rb[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            f32x4 acc = zero4();
#pragma unroll
            for (int tj = 0; tj <= ti; ++tj) acc = Elem<ST>::mma(acc, frag_rows(sT, LD, 16 * ti, 16 * tj), Yb[tj]);
            R[ti] = acc;
            Rb[ti] = Elem<ST>::pack(acc);
        }
        if constexpr (!SUMMARY) {
            // O = scale Gamma (Q S^T) + P R
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) acc = Elem<ST>::mma(acc, frag_rows(sQ, LDK, 16 * ti, 16 * kb), Sb[kb]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= scale * sC[16 * ti + 4 * lg + r];
#pragma unroll
                for (int tj = 0; tj <= ti; ++tj) acc = Elem<ST>::mma(acc, frag_rows(sP, LD, 16 * ti, 16 * tj), Rb[tj]);
                if (vrow) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * ti + 4 * lg + r;
                        if (t < L) out[((size_t)(b * T + t0 + t) * H + h) * V + myrow] = Elem<ST>::from_f(acc[r]);
                    }
                }
            }
        }
        // S <- Gamma_L S + K^T (e R)
        frag ERb[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 er;
#pragma unroll
            for (int r = 0; r < 4; ++r) er[r] = sC[64 + 16 * tb + 4 * lg + r] * R[tb][r];
            ERb[tb] = Elem<ST>::pack(er);
        }
        const float gl = sC[192];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x4 acc = S[kb] * gl;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) acc = Elem<ST>::mma(acc, frag_rows(sKT, LD, 16 * kb, 16 * tb), ERb[tb]);
            S[kb] = acc;
        }
        (void)L;
    }

    // exit state
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
        const int kk = 16 * kb + 4 * lg;
        if (vrow) {
            if (ht) *reinterpret_cast<f32x4*>(ht + (((size_t)n * H + h) * V + myrow) * KD + kk) = S[kb];
        } else if constexpr (SUMMARY) {
            *reinterpret_cast<f32x4*>(Mout + (((size_t)n * H + h) * KD + (myrow - V)) * KD + kk) = S[kb];
        }
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_chunk_table(const int32_t* cu, int N, int chunk, long cap, int* chunk_off,
                              int2* table, hipStream_t s) {
    timing_begin("chunk_table", s);
    chunk_table_kernel<<<1, 256, 0, s>>>(cu, N, chunk, (int)cap, chunk_off, table);
    timing_end(s);
    return hipGetLastError();
}

template <typename ST, int KD>
static hipError_t run_gdn(int mode, const ST* q, const ST* k, const ST* v, const float* g,
                          const float* beta, const float* h0, const int32_t* cu,
                          const GdnWorkspace& ws, int N, int B, int T, int H, int HK, int V,
                          float scale, ST* out, float* ht, float* Mout, hipStream_t s) {
    const bool packed = cu != nullptr;
    const long slots = gdn_slots(B, T, N, packed);
    const int nc = (T + GC - 1) / GC;
    hipError_t err;
    if (packed) {
        err = launch_chunk_table(cu, N, GC, slots, ws.chunk_off, ws.table, s);
        if (err != hipSuccess) return err;
    }
    if (slots > 0) {
        timing_begin("gdn_prep", s);
        gdn_prep_kernel<ST, KD><<<dim3((unsigned)slots, H), 256, 0, s>>>(
            q, k, g, beta, packed ? ws.table : nullptr, cu, T, H, HK, nc, scale, mode == 0 ? 1 : 0,
            ws.factors);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    constexpr int NW = 4;
    const int rows = mode == 0 ? V : V + KD;
    const int nvb = rows / (16 * NW);
    const int chains = N * H;
    const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvb);
    if (chains == 0) return hipSuccess;
    if (mode == 0) {
        timing_begin("gdn_chain", s);
        gdn_chain_kernel<ST, KD, NW, false><<<grid, 64 * NW, 0, s>>>(
            q, k, v, h0, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, nvb, scale, out, ht, nullptr);
    } else {
        timing_begin("gdn_summary_chain", s);
        gdn_chain_kernel<ST, KD, NW, true><<<grid, 64 * NW, 0, s>>>(
            q, k, v, nullptr, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, nvb, scale, nullptr, ht, Mout);
    }
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_gdn(bool bf16, int mode, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const float* h0, const int32_t* cu,
                      const GdnWorkspace& ws, int N, int B, int T, int H, int HK, int K, int V,
                      float scale, void* out, float* ht, float* Mout, hipStream_t s) {
    if (bf16) {
        const bf16_t *qq = (const bf16_t*)q, *kk = (const bf16_t*)k, *vv = (const bf16_t*)v;
        if (K == 128) return run_gdn<bf16_t, 128>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (bf16_t*)out, ht, Mout, s);
        return run_gdn<bf16_t, 64>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (bf16_t*)out, ht, Mout, s);
    }
    const float *qq = (const float*)q, *kk = (const float*)k, *vv = (const float*)v;
    if (K == 128) return run_gdn<float, 128>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (float*)out, ht, Mout, s);
    return run_gdn<float, 64>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (float*)out, ht, Mout, s);
}

}  // namespace sf

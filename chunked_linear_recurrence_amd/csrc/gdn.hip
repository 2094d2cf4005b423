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
//   [0,64) Gamma_t  [64,128) e_t  [128,192) beta_t  [192,256) G_t
// (Gamma_L = Gamma_63: padded tokens of a partial chunk have zero gate)
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
        gC[192 + tid] = G;
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
// Pre, bf16: one wavefront per (chunk slot, head), no workgroup barriers.
//  - K and Q rows go straight from global memory into 16x16x32 MFMA
//    fragments (lane (n, g) holds row 16R+n, columns 32p+8g..+7), which serve
//    as both operands of K K^T and Q K^T on the 10 lower 16x16 tiles.
//  - A = diag(beta)(strictly lower D o K K^T) is kept in LDS as packed
//    columns (column i holds rows i+1..63, 16-byte aligned).
//  - T = (I + A)^-1 by forward substitution with one column per lane
//    (T[t][j] = 1{t == j} - sum_{i<t} A[t][i] T[i][j]), applied right-looking:
//    A's columns are read as broadcasts from LDS, T's column stays in 64
//    registers.
//  - T and P leave through a 64x64 bf16 LDS staging tile with 16-byte stores.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int tri_off(int t) {  // sum_{s<t} round_up(s, 4)
    return 8 * (t / 4) * (t / 4) + 4 * (t / 4) + ((t % 4) ? 4 * (t / 4) * (t % 4) + 4 * ((t % 4) - 1) : 0);
}
// Column i of the strictly lower 64x64 A (rows i+1..63) starts at col_off(i),
// each column padded to a multiple of 4 floats: sum_{i'<i} round_up(63 - i', 4).
__host__ __device__ constexpr int col_off(int i) { return tri_off(GC) - tri_off(GC - i); }

template <int KD, bool WANT_P>
__global__ __launch_bounds__(64) void gdn_prep_wave_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                           const float* __restrict__ g,
                                                           const float* __restrict__ beta,
                                                           const int2* __restrict__ table,
                                                           const int32_t* __restrict__ cu, int T, int H,
                                                           int HK, int nc, int n_slots, float scale,
                                                           uint8_t* __restrict__ fac) {
    constexpr int KP = KD / 32;
    constexpr int NPW = 1;
    __shared__ __align__(16) float sA[tri_off(GC)];
    __shared__ __align__(16) bf16_t sO[GC * GC];
    __shared__ float sG[GC], sB[GC];

    const int h = blockIdx.y;
    const int hk = h / (H / HK);
    const int lane = threadIdx.x, ln = lane & 15, lg = lane >> 4;
    const bf16x8 zero8 = {};

    bf16x8 kf[4][KP], qf[4][KP];
    float gv, bv;
    int b, t0, L;
    auto load = [&](int slot) __attribute__((always_inline)) {
        const int t_lane = min(lane, L - 1);
        const size_t gi = (size_t)(b * T + t0 + t_lane) * H + h;
        gv = lane < L ? g[gi] : 0.f;
        bv = lane < L ? beta[gi] : 0.f;
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            const int t = 16 * R + ln;
            const size_t row = ((size_t)(b * T + t0 + min(t, L - 1)) * HK + hk) * KD;
#pragma unroll
            for (int p = 0; p < KP; ++p) {
                const bf16x8 kv = *reinterpret_cast<const bf16x8*>(k + row + 32 * p + 8 * lg);
                kf[R][p] = t < L ? kv : zero8;
                if constexpr (WANT_P) {
                    const bf16x8 qv = *reinterpret_cast<const bf16x8*>(q + row + 32 * p + 8 * lg);
                    qf[R][p] = t < L ? qv : zero8;
                }
            }
        }
        (void)slot;
    };

    int slot = blockIdx.x * NPW;
    if (slot >= n_slots || !chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    load(slot);
    for (int s = 0; s < NPW; ++s, ++slot) {
        // gates of this slot (registers loaded with the slot's K/Q)
        const float G = wave_inclusive_scan(gv);
        sG[lane] = G;
        sB[lane] = bv;
        uint8_t* rec = fac + ((size_t)slot * H + h) * gdn_factor_bytes(2);
        bf16_t* gT = reinterpret_cast<bf16_t*>(rec);
        bf16_t* gP = gT + GC * GC;
        float* gC = reinterpret_cast<float*>(gP + GC * GC);
        {
            const float GL = __shfl(G, 63, 64);
            gC[lane] = expf(G);
            gC[64 + lane] = expf(GL - G);
            gC[128 + lane] = bv;
            gC[192 + lane] = G;
        }
#pragma unroll
        for (int i = 0; i < GC * GC / 8 / 64; ++i) *reinterpret_cast<u128*>(sO + 8 * (lane + 64 * i)) = u128{0u, 0u, 0u, 0u};
        __syncthreads();

#pragma unroll
        for (int tt = 0; tt < 10; ++tt) {
            const int ti = (tt >= 1) + (tt >= 3) + (tt >= 6);
            const int tj = tt - ti * (ti + 1) / 2;
            f32x4 a = zero4(), pq = zero4();
#pragma unroll
            for (int p = 0; p < KP; ++p) {
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ti][p], kf[tj][p], a, 0, 0, 0);
                if constexpr (WANT_P) pq = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ti][p], kf[tj][p], pq, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * ti + 4 * lg + r, i = 16 * tj + ln;
                const float d = expf(fminf(sG[t] - sG[i], 0.f));
                if (i < t) sA[col_off(i) + (t - i - 1)] = sB[t] * d * a[r];
                if (WANT_P && i <= t) sO[t * GC + i] = f2bf(scale * d * pq[r]);
            }
        }
        __syncthreads();
        if constexpr (WANT_P) {
#pragma unroll
            for (int i = 0; i < GC * GC / 8 / 64; ++i) {
                const int u = lane + 64 * i;
                *reinterpret_cast<u128*>(gP + 8 * u) = *reinterpret_cast<const u128*>(sO + 8 * u);
            }
        }
        // next slot's loads go out now (the fragment registers are free) and land during the solve
        const bool next = s + 1 < NPW && slot + 1 < n_slots && chunk_coords(slot + 1, table, cu, T, nc, b, t0, L);
        if (next) load(slot + 1);

        // forward substitution, lane = column j of T, right-looking: once row t
        // of the column is final, its contribution A[r][t] x_t leaves every later
        // row r, so each step is 63 - t independent FMAs; the next column of A
        // is read from LDS while the current one is applied
        float x[GC];
#pragma unroll
        for (int r = 0; r < GC; ++r) x[r] = (r == lane) ? 1.f : 0.f;
        f32x4 cur[16], nxt[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) cur[m] = *reinterpret_cast<const f32x4*>(sA + col_off(0) + 4 * m);
#pragma unroll
        for (int t = 0; t < GC - 1; ++t) {
            const int n = GC - 1 - t, n1 = n - 1;  // entries in column t and t+1
#pragma unroll
            for (int m = 0; m < (n1 + 3) / 4; ++m) nxt[m] = *reinterpret_cast<const f32x4*>(sA + col_off(t + 1) + 4 * m);
            const float xt = x[t];
#pragma unroll
            for (int m = 0; m < (n + 3) / 4; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * m + e < n) x[t + 1 + 4 * m + e] -= cur[m][e] * xt;
#pragma unroll
            for (int m = 0; m < 16; ++m) cur[m] = nxt[m];
        }
        __syncthreads();  // staging tile free again (P copy done)
#pragma unroll
        for (int t = 0; t < GC; ++t) sO[t * GC + lane] = f2bf(x[t]);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < GC * GC / 8 / 64; ++i) {
            const int u = lane + 64 * i;
            *reinterpret_cast<u128*>(gT + 8 * u) = *reinterpret_cast<const u128*>(sO + 8 * u);
        }
        if (!next) break;
        __syncthreads();  // sG/sB/sA/sO are rewritten for the next slot
    }
}

// ---------------------------------------------------------------------------
// ST + Out: one workgroup = NW wavefronts = 16*NW state rows of one chain.
// ---------------------------------------------------------------------------
template <typename ST>
__device__ __forceinline__ ST unit_elem(const u128& u, int e) {
    if constexpr (sizeof(ST) == 2) {
        const uint32_t w = u[e >> 1];
        return (ST)((e & 1) ? (w >> 16) : (w & 0xffffu));
    } else {
        return __uint_as_float(u[e]);
    }
}

template <typename ST, int KD, bool SUMMARY>
struct ChainSmem {
    static constexpr int E = 16 / sizeof(ST);
    static constexpr int LDK = KD + E, LD = GC + E;
    // one staging buffer: K [64][LDK], K^T [KD][LD], T [64][LD], coef float[256],
    // and (forward only) Q [64][LDK], P [64][LD]
    static constexpr int OFF_K = 0;
    static constexpr int OFF_KT = OFF_K + GC * LDK * (int)sizeof(ST);
    static constexpr int OFF_T = OFF_KT + KD * LD * (int)sizeof(ST);
    static constexpr int OFF_C = OFF_T + GC * LD * (int)sizeof(ST);
    static constexpr int OFF_Q = OFF_C + 256 * 4;
    static constexpr int OFF_P = OFF_Q + (SUMMARY ? 0 : GC * LDK * (int)sizeof(ST));
    static constexpr int BYTES = OFF_P + (SUMMARY ? 0 : GC * LD * (int)sizeof(ST));
    static constexpr int NBUF = 2 * BYTES <= 160 * 1024 - 1024 ? 2 : 1;
};

template <typename ST, int KD, int NW, bool SUMMARY>
__global__ __launch_bounds__(64 * NW) void gdn_chain_kernel(
    const ST* __restrict__ q, const ST* __restrict__ k, const ST* __restrict__ v,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const uint8_t* __restrict__ fac, int T, int H, int HK, int V, int n_seq, int nc, int nvb,
    float scale, ST* __restrict__ out, float* __restrict__ ht, float* __restrict__ Mout) {
    typedef ChainSmem<ST, KD, SUMMARY> SM;
    constexpr int E = SM::E, LDK = SM::LDK, LD = SM::LD, NBUF = SM::NBUF;
    constexpr int NT = 64 * NW;
    constexpr int KB = KD / 16;
    constexpr int UPR = KD / E;             // units per K/Q row
    constexpr int NUK = GC * UPR;           // units per K (or Q) chunk
    constexpr int NUT = GC * GC / E;        // units per T (or P) block
    constexpr int PK = NUK / NT;
    constexpr int PT = NUT / NT;
    static_assert(NUK % NT == 0 && NUT % NT == 0, "staging units must divide evenly");
    typedef typename Elem<ST>::frag frag;

    __shared__ __align__(16) uint8_t smem[NBUF * SM::BYTES];

    int chain, vb;
    xcd_split(blockIdx.x, nvb, chain, vb);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, hk = h / (H / HK);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int myrow = (vb * NW + wave) * 16 + ln;
    const bool vrow = myrow < V;
    const int vload_row = vrow ? myrow : 0;

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

    // Staging registers live only within one iteration: loads for chunk c+1
    // are issued before chunk c's products and written to the other LDS
    // buffer after them, so their latency hides behind the compute. Loads use
    // clamped (valid) rows; rows past the chunk end are zeroed on the write.
    u128 rk[PK], rq[PK], rt[PT], rp[PT], rc;
    ST rv[16];
    auto issue = [&](int c) __attribute__((always_inline)) {
        const int t0 = bos + c * GC, L = min(GC, eos - t0);
        const uint8_t* rec = fac + ((size_t)(slot0 + c) * H + h) * rec_bytes;
        const ST* gT = reinterpret_cast<const ST*>(rec);
        const ST* gP = gT + GC * GC;
        const float* gC = reinterpret_cast<const float*>(gP + GC * GC);
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int u = tid + i * NT;
            const int t = min(u / UPR, L - 1), col = (u % UPR) * E;
            const size_t off = ((size_t)(b * T + t0 + t) * HK + hk) * KD + col;
            rk[i] = *reinterpret_cast<const u128*>(k + off);
            if constexpr (!SUMMARY) rq[i] = *reinterpret_cast<const u128*>(q + off);
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + i * NT;
            rt[i] = *reinterpret_cast<const u128*>(gT + u * E);
            if constexpr (!SUMMARY) rp[i] = *reinterpret_cast<const u128*>(gP + u * E);
        }
        rc = *reinterpret_cast<const u128*>(gC + 4 * lane);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = min(16 * (i >> 2) + 4 * lg + (i & 3), L - 1);
            rv[i] = v[((size_t)(b * T + t0 + t) * H + h) * V + vload_row];
        }
    };
    float vv[16];
    auto commit = [&](int c, int buf) __attribute__((always_inline)) {
        const int L = min(GC, eos - (bos + c * GC));
        uint8_t* base = smem + buf * SM::BYTES;
        ST* sK = reinterpret_cast<ST*>(base + SM::OFF_K);
        ST* sKT = reinterpret_cast<ST*>(base + SM::OFF_KT);
        ST* sT = reinterpret_cast<ST*>(base + SM::OFF_T);
        float* sC = reinterpret_cast<float*>(base + SM::OFF_C);
        ST* sQ = reinterpret_cast<ST*>(base + SM::OFF_Q);
        ST* sP = reinterpret_cast<ST*>(base + SM::OFF_P);
        const u128 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int u = tid + i * NT;
            const int t = u / UPR, col = (u % UPR) * E;
            const u128 kv = t < L ? rk[i] : zero;
            *reinterpret_cast<u128*>(sK + t * LDK + col) = kv;
#pragma unroll
            for (int e = 0; e < E; ++e) sKT[(col + e) * LD + t] = unit_elem<ST>(kv, e);
            if constexpr (!SUMMARY) *reinterpret_cast<u128*>(sQ + t * LDK + col) = t < L ? rq[i] : zero;
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = tid + i * NT;
            const int r = u / (GC / E), col = (u % (GC / E)) * E;
            *reinterpret_cast<u128*>(sT + r * LD + col) = rt[i];
            if constexpr (!SUMMARY) *reinterpret_cast<u128*>(sP + r * LD + col) = rp[i];
        }
        if (wave == 0) *reinterpret_cast<u128*>(sC + 4 * lane) = rc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int t = 16 * (i >> 2) + 4 * lg + (i & 3);
            vv[i] = (vrow && t < L) ? Elem<ST>::to_f(rv[i]) : 0.f;
        }
    };

    if (nch > 0) {
        issue(0);
        commit(0, 0);
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int t0 = bos + c * GC, L = min(GC, eos - t0);
        const int buf = NBUF == 2 ? (c & 1) : 0;
        const uint8_t* base = smem + buf * SM::BYTES;
        const ST* sK = reinterpret_cast<const ST*>(base + SM::OFF_K);
        const ST* sKT = reinterpret_cast<const ST*>(base + SM::OFF_KT);
        const ST* sT = reinterpret_cast<const ST*>(base + SM::OFF_T);
        const float* sC = reinterpret_cast<const float*>(base + SM::OFF_C);
        const ST* sQ = reinterpret_cast<const ST*>(base + SM::OFF_Q);
        const ST* sP = reinterpret_cast<const ST*>(base + SM::OFF_P);
        const bool more = c + 1 < nch;
        if (more) issue(c + 1);
        float vcur[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) vcur[i] = vv[i];

        frag Sb[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) Sb[kb] = Elem<ST>::pack(S[kb]);

        // X = K S^T ; Y = beta (V - Gamma X)
        frag Yb[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; kb += 2)
                acc = Elem<ST>::mma2(acc, frag_rows(sK, LDK, 16 * tb, 16 * kb), frag_rows(sK, LDK, 16 * tb, 16 * kb + 16),
                                     Sb[kb], Sb[kb + 1]);
            f32x4 y;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * tb + 4 * lg + r;
                y[r] = sC[128 + t] * (vcur[4 * tb + r] - sC[t] * acc[r]);
            }
            Yb[tb] = Elem<ST>::pack(y);
        }
        // R = T Y (T is lower triangular; its upper 16x16 blocks are stored as zeros)
        f32x4 R[4];
        frag Rb[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            f32x4 acc = zero4();
#pragma unroll
            for (int tj = 0; tj <= ti; tj += 2)
                acc = Elem<ST>::mma2(acc, frag_rows(sT, LD, 16 * ti, 16 * tj), frag_rows(sT, LD, 16 * ti, 16 * tj + 16),
                                     Yb[tj], Yb[tj + 1]);
            R[ti] = acc;
            Rb[ti] = Elem<ST>::pack(acc);
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
        const float gl = sC[63];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f32x4 acc = S[kb] * gl;
#pragma unroll
            for (int tb = 0; tb < 4; tb += 2)
                acc = Elem<ST>::mma2(acc, frag_rows(sKT, LD, 16 * kb, 16 * tb), frag_rows(sKT, LD, 16 * kb, 16 * tb + 16),
                                     ERb[tb], ERb[tb + 1]);
            S[kb] = acc;
        }
        if constexpr (!SUMMARY) {
            // O = scale Gamma (Q S^T) + P R  (S^T here is the chunk-entry state, Sb)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; kb += 2)
                    acc = Elem<ST>::mma2(acc, frag_rows(sQ, LDK, 16 * ti, 16 * kb), frag_rows(sQ, LDK, 16 * ti, 16 * kb + 16),
                                         Sb[kb], Sb[kb + 1]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= scale * sC[16 * ti + 4 * lg + r];
#pragma unroll
                for (int tj = 0; tj <= ti; tj += 2)
                    acc = Elem<ST>::mma2(acc, frag_rows(sP, LD, 16 * ti, 16 * tj), frag_rows(sP, LD, 16 * ti, 16 * tj + 16),
                                         Rb[tj], Rb[tj + 1]);
                if (vrow) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * ti + 4 * lg + r;
                        if (t < L) out[((size_t)(b * T + t0 + t) * H + h) * V + myrow] = Elem<ST>::from_f(acc[r]);
                    }
                }
            }
        }
        if (more) {
            if constexpr (NBUF == 1) __syncthreads();
            commit(c + 1, NBUF == 2 ? (buf ^ 1) : 0);
        }
        __syncthreads();
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
// ST + Out, bf16, warp-specialised: one workgroup = one 16-row state slice of
// one chain, KS compute wavefronts + 4 loader wavefronts.
//
//  - Compute wavefront j owns the state columns k in k-tiles [j KB/KS, (j+1) KB/KS)
//    (float32 MFMA accumulators) and the tokens of t-tiles [j 4/KS, (j+1) 4/KS).
//    The bf16 copy of the whole slice state is exchanged through LDS, so each
//    wavefront forms X = K S^T and Q S^T for its own tokens over all k; the
//    corrected values Y of all tokens are exchanged the same way; R = T Y is
//    formed redundantly by every compute wavefront (6 MFMAs), which then
//    updates its own state columns and writes its own output tokens.
//  - Loader wavefronts move chunk c+1 (K, Q, T, P, coefficients, the slice's V)
//    from global memory into the other half of a double-buffered LDS stage
//    and write chunk c-1's output tile to global memory with 16-byte stores,
//    so the compute wavefronts never wait on vector memory. K^T fragments for
//    the state update are read from the natural K tile with the transposing
//    LDS read.
//  Two workgroup barriers per chunk separate the exchange phases.
// ---------------------------------------------------------------------------
template <int KD, bool SUMMARY>
struct WsSmem {
    static constexpr int E = 8;  // bf16 per 16-byte unit
    static constexpr int LDK = KD + E, LD = GC + E, LDO = 16 + E;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_T = OFF_K + GC * LDK * 2;
    static constexpr int OFF_C = OFF_T + GC * LD * 2;
    static constexpr int OFF_V = OFF_C + 256 * 4;
    static constexpr int OFF_Q = OFF_V + 16 * LD * 2;
    static constexpr int OFF_P = OFF_Q + (SUMMARY ? 0 : GC * LDK * 2);
    static constexpr int BUF = OFF_P + (SUMMARY ? 0 : GC * LD * 2);
    static constexpr int OFF_S = 2 * BUF;                       // state frags [KB][64] x 8 B
    static constexpr int OFF_Y = OFF_S + (KD / 16) * 64 * 8;    // Y frags [4][64] x 8 B
    static constexpr int OFF_O = OFF_Y + 4 * 64 * 8;            // output tiles [2][64][LDO] bf16
    static constexpr int BYTES = OFF_O + (SUMMARY ? 0 : 2 * GC * LDO * 2);
};

template <int KD, int KS, bool SUMMARY>
__global__ __launch_bounds__(64 * (KS + 4)) void gdn_chain_ws_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const uint8_t* __restrict__ fac, int T, int H, int HK, int V, int n_seq, int nc, int nvb,
    float scale, bf16_t* __restrict__ out, float* __restrict__ ht, float* __restrict__ Mout) {
    typedef WsSmem<KD, SUMMARY> SM;
    typedef Elem<bf16_t> El;
    typedef El::frag frag;
    constexpr int E = SM::E, LDK = SM::LDK, LD = SM::LD, LDO = SM::LDO;
    constexpr int KB = KD / 16;
    constexpr int KT = KB / KS;       // state k-tiles per compute wavefront
    constexpr int TT = 4 / KS;        // token tiles per compute wavefront
    constexpr int NLT = 256;          // loader threads
    constexpr int UPR = KD / E;
    constexpr int NUK = GC * UPR;
    constexpr int NUT = GC * GC / E;
    constexpr int PK = NUK / NLT, PT = NUT / NLT;
    static_assert(KB % KS == 0 && 4 % KS == 0 && NUK % NLT == 0 && NUT % NLT == 0, "tiling");

    __shared__ __align__(16) uint8_t smem[SM::BYTES];
    i16x4* sS = reinterpret_cast<i16x4*>(smem + SM::OFF_S);
    i16x4* sY = reinterpret_cast<i16x4*>(smem + SM::OFF_Y);

    int chain, vb;
    xcd_split(blockIdx.x, nvb, chain, vb);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, hk = h / (H / HK);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const bool loader = wave >= KS;
    const int row0 = 16 * vb;               // first state row of this slice
    const bool vrows = row0 < V;            // value rows (else transition rows, summary only)

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
    const size_t rec_bytes = gdn_factor_bytes(2);
    auto buf_ptr = [&](int c) __attribute__((always_inline)) { return smem + (c & 1) * SM::BUF; };

    // ---------------- loader role ----------------
    const int lt = tid - 64 * KS;
    u128 rk[PK], rq[PK], rt[PT], rp[PT], rc, rvv;
    auto issue = [&](int c) __attribute__((always_inline)) {
        const int t0 = bos + c * GC, L = min(GC, eos - t0);
        const uint8_t* rec = fac + ((size_t)(slot0 + c) * H + h) * rec_bytes;
        const bf16_t* gT = reinterpret_cast<const bf16_t*>(rec);
        const bf16_t* gP = gT + GC * GC;
        const float* gC = reinterpret_cast<const float*>(gP + GC * GC);
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int u = lt + i * NLT;
            const int t = min(u / UPR, L - 1), col = (u % UPR) * E;
            const size_t off = ((size_t)(b * T + t0 + t) * HK + hk) * KD + col;
            rk[i] = *reinterpret_cast<const u128*>(k + off);
            if constexpr (!SUMMARY) rq[i] = *reinterpret_cast<const u128*>(q + off);
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = lt + i * NLT;
            rt[i] = *reinterpret_cast<const u128*>(gT + u * E);
            if constexpr (!SUMMARY) rp[i] = *reinterpret_cast<const u128*>(gP + u * E);
        }
        if (lt < 64) rc = *reinterpret_cast<const u128*>(gC + 4 * lt);
        if (vrows && lt < 128) {
            const int t = min(lt >> 1, L - 1), col = (lt & 1) * E;
            rvv = *reinterpret_cast<const u128*>(v + ((size_t)(b * T + t0 + t) * H + h) * V + row0 + col);
        }
    };
    auto commit = [&](int c) __attribute__((always_inline)) {
        const int L = min(GC, eos - (bos + c * GC));
        uint8_t* base = buf_ptr(c);
        bf16_t* sK = reinterpret_cast<bf16_t*>(base + SM::OFF_K);
        bf16_t* sT = reinterpret_cast<bf16_t*>(base + SM::OFF_T);
        float* sC = reinterpret_cast<float*>(base + SM::OFF_C);
        bf16_t* sVT = reinterpret_cast<bf16_t*>(base + SM::OFF_V);
        bf16_t* sQ = reinterpret_cast<bf16_t*>(base + SM::OFF_Q);
        bf16_t* sP = reinterpret_cast<bf16_t*>(base + SM::OFF_P);
        const u128 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int u = lt + i * NLT;
            const int t = u / UPR, col = (u % UPR) * E;
            *reinterpret_cast<u128*>(sK + t * LDK + col) = t < L ? rk[i] : zero;
            if constexpr (!SUMMARY) *reinterpret_cast<u128*>(sQ + t * LDK + col) = t < L ? rq[i] : zero;
        }
#pragma unroll
        for (int i = 0; i < PT; ++i) {
            const int u = lt + i * NLT;
            const int r = u / (GC / E), col = (u % (GC / E)) * E;
            *reinterpret_cast<u128*>(sT + r * LD + col) = rt[i];
            if constexpr (!SUMMARY) *reinterpret_cast<u128*>(sP + r * LD + col) = rp[i];
        }
        if (lt < 64) *reinterpret_cast<u128*>(sC + 4 * lt) = rc;
        if (lt < 128) {
            const int t = lt >> 1, col = (lt & 1) * E;
            const u128 x = (vrows && t < L) ? rvv : zero;
#pragma unroll
            for (int e = 0; e < E; ++e) sVT[(col + e) * LD + t] = unit_elem<bf16_t>(x, e);
        }
    };
    auto store_out = [&](int c) __attribute__((always_inline)) {  // output tile of chunk c from LDS to global
        if constexpr (!SUMMARY) {
            const int t0 = bos + c * GC, L = min(GC, eos - t0);
            const bf16_t* sO = reinterpret_cast<const bf16_t*>(smem + SM::OFF_O) + (c & 1) * GC * LDO;
            if (lt < 128) {
                const int t = lt >> 1, col = (lt & 1) * E;
                if (t < L)
                    *reinterpret_cast<u128*>(out + ((size_t)(b * T + t0 + t) * H + h) * V + row0 + col) =
                        *reinterpret_cast<const u128*>(sO + t * LDO + col);
            }
        }
    };

    // ---------------- compute role ----------------
    const int j = wave;  // compute wavefront index (valid when !loader)
    f32x4 S[KT];
    if (!loader) {
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            const int kt = j * KT + i, kk = 16 * kt + 4 * lg;
            const int row = row0 + ln;
            if constexpr (!SUMMARY) {
                S[i] = h0 ? *reinterpret_cast<const f32x4*>(h0 + (((size_t)n * H + h) * V + row) * KD + kk) : zero4();
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[i][r] = (!vrows && kk + r == row - V) ? 1.f : 0.f;
            }
            sS[kt * 64 + lane] = El::pack(S[i]);
        }
    } else if (nch > 0) {
        issue(0);
        commit(0);
        if (nch > 1) issue(1);  // in flight across the first iteration
    }
    __syncthreads();

    f32x4 QS[TT];
    for (int c = 0; c < nch; ++c) {
        const int t0 = bos + c * GC, L = min(GC, eos - t0);
        const uint8_t* base = buf_ptr(c);
        const bf16_t* sK = reinterpret_cast<const bf16_t*>(base + SM::OFF_K);
        const bf16_t* sT = reinterpret_cast<const bf16_t*>(base + SM::OFF_T);
        const float* sC = reinterpret_cast<const float*>(base + SM::OFF_C);
        const bf16_t* sVT = reinterpret_cast<const bf16_t*>(base + SM::OFF_V);
        const bf16_t* sQ = reinterpret_cast<const bf16_t*>(base + SM::OFF_Q);
        const bf16_t* sP = reinterpret_cast<const bf16_t*>(base + SM::OFF_P);
        const bool more = c + 1 < nch;
        // ---- phase 1: X = K S^T and Q S^T for own tokens, Y = beta (V - Gamma X) ----
        if (loader) {
            if (c > 0) store_out(c - 1);
        } else {
            // every LDS operand of the phase is read before the first product
            frag Sf[KB], Kf[TT][KB], Qf[TT][KB], Vf[TT];
            f32x4 gam[TT], bet[TT];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) Sf[kb] = sS[kb * 64 + lane];
#pragma unroll
            for (int i = 0; i < TT; ++i) {
                const int tt = j * TT + i;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    Kf[i][kb] = frag_rows(sK, LDK, 16 * tt, 16 * kb);
                    if constexpr (!SUMMARY) Qf[i][kb] = frag_rows(sQ, LDK, 16 * tt, 16 * kb);
                }
                Vf[i] = frag_rows(sVT, LD, 0, 16 * tt);
                gam[i] = *reinterpret_cast<const f32x4*>(sC + 16 * tt + 4 * lg);
                bet[i] = *reinterpret_cast<const f32x4*>(sC + 128 + 16 * tt + 4 * lg);
            }
#pragma unroll
            for (int i = 0; i < TT; ++i) {
                const int tt = j * TT + i;
                f32x4 x = zero4(), qs = zero4();
#pragma unroll
                for (int kb = 0; kb < KB; kb += 2) {
                    x = El::mma2(x, Kf[i][kb], Kf[i][kb + 1], Sf[kb], Sf[kb + 1]);
                    if constexpr (!SUMMARY) qs = El::mma2(qs, Qf[i][kb], Qf[i][kb + 1], Sf[kb], Sf[kb + 1]);
                }
                QS[i] = qs * gam[i] * scale;
                const f32x4 vx = El::unpack(Vf[i]);
                sY[tt * 64 + lane] = El::pack(bet[i] * (vx - gam[i] * x));
            }
        }
        __syncthreads();
        // ---- phase 2: R = T Y, state update of own columns, own output tokens ----
        if (loader) {
            // chunk c+1 was issued one iteration ago; chunk c+2 stays in flight for the next one
            if (more) commit(c + 1);
            if (c + 2 < nch) issue(c + 2);
        } else {
            frag Yf[4], Tf[6][2], Ka[KT][2][2], Pf[TT][2][2];
            f32x4 ec[4];
            constexpr int TI[6] = {0, 1, 2, 2, 3, 3}, TJ[6] = {0, 0, 0, 2, 0, 2};
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                Yf[ti] = sY[ti * 64 + lane];
                ec[ti] = *reinterpret_cast<const f32x4*>(sC + 64 + 16 * ti + 4 * lg);
            }
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                Tf[p][0] = frag_rows(sT, LD, 16 * TI[p], 16 * TJ[p]);
                Tf[p][1] = frag_rows(sT, LD, 16 * TI[p], 16 * TJ[p] + 16);
            }
            // K^T fragments of own state columns, read transposed from the natural K tile
#pragma unroll
            for (int i = 0; i < KT; ++i)
#pragma unroll
                for (int tp = 0; tp < 2; ++tp) {
                    Ka[i][tp][0] = frag_rows_t(sK, LDK, 32 * tp, 16 * (j * KT + i));
                    Ka[i][tp][1] = frag_rows_t(sK, LDK, 32 * tp + 16, 16 * (j * KT + i));
                }
            if constexpr (!SUMMARY) {
#pragma unroll
                for (int i = 0; i < TT; ++i) {
                    const int tt = j * TT + i;
                    // all four 16-token blocks of the row; P's upper blocks are stored as zeros
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) {
                        Pf[i][pp][0] = frag_rows(sP, LD, 16 * tt, 32 * pp);
                        Pf[i][pp][1] = frag_rows(sP, LD, 16 * tt, 32 * pp + 16);
                    }
                }
            }
            const float gl = sC[63];
            f32x4 R[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
            for (int p = 0; p < 6; ++p)
                R[TI[p]] = El::mma2(R[TI[p]], Tf[p][0], Tf[p][1], Yf[TJ[p]], Yf[TJ[p] + 1]);
            frag Rb[4], ER[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                Rb[ti] = El::pack(R[ti]);
                ER[ti] = El::pack(R[ti] * ec[ti]);
            }
            // own state columns: S^T[kt] <- Gamma_L S^T[kt] + K^T[kt, :] (e R)
#pragma unroll
            for (int i = 0; i < KT; ++i) {
                f32x4 acc = S[i] * gl;
                acc = El::mma2(acc, Ka[i][0][0], Ka[i][0][1], ER[0], ER[1]);
                acc = El::mma2(acc, Ka[i][1][0], Ka[i][1][1], ER[2], ER[3]);
                S[i] = acc;
            }
            if constexpr (!SUMMARY) {
                bf16_t* sO = reinterpret_cast<bf16_t*>(smem + SM::OFF_O) + (c & 1) * GC * LDO;
#pragma unroll
                for (int i = 0; i < TT; ++i) {
                    const int tt = j * TT + i;
                    f32x4 acc = QS[i];
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp) acc = El::mma2(acc, Pf[i][pp][0], Pf[i][pp][1], Rb[2 * pp], Rb[2 * pp + 1]);
                    const frag o = El::pack(acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) sO[(16 * tt + 4 * lg + r) * LDO + ln] = (bf16_t)o[r];
                }
            }
#pragma unroll
            for (int i = 0; i < KT; ++i) sS[(j * KT + i) * 64 + lane] = El::pack(S[i]);
        }
        __syncthreads();
        (void)L;
        (void)t0;
    }
    if (loader) {
        if (nch > 0) store_out(nch - 1);
    } else {
#pragma unroll
        for (int i = 0; i < KT; ++i) {
            const int kt = j * KT + i, kk = 16 * kt + 4 * lg, row = row0 + ln;
            if (vrows) {
                if (ht) *reinterpret_cast<f32x4*>(ht + (((size_t)n * H + h) * V + row) * KD + kk) = S[i];
            } else if constexpr (SUMMARY) {
                *reinterpret_cast<f32x4*>(Mout + (((size_t)n * H + h) * KD + (row - V)) * KD + kk) = S[i];
            }
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
        if constexpr (sizeof(ST) == 2) {
            const unsigned gx = (unsigned)slots;
            if (mode == 0)
                gdn_prep_wave_kernel<KD, true><<<dim3(gx, H), 64, 0, s>>>(
                    q, k, g, beta, packed ? ws.table : nullptr, cu, T, H, HK, nc, (int)slots, scale, ws.factors);
            else
                gdn_prep_wave_kernel<KD, false><<<dim3(gx, H), 64, 0, s>>>(
                    q, k, g, beta, packed ? ws.table : nullptr, cu, T, H, HK, nc, (int)slots, scale, ws.factors);
        } else
            gdn_prep_kernel<ST, KD><<<dim3((unsigned)slots, H), 256, 0, s>>>(
                q, k, g, beta, packed ? ws.table : nullptr, cu, T, H, HK, nc, scale, mode == 0 ? 1 : 0,
                ws.factors);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const int rows = mode == 0 ? V : V + KD;
    const int chains = N * H;
    if (chains == 0) return hipSuccess;
    if constexpr (sizeof(ST) == 2) {
        constexpr int KS = 4;
        const int nvb = rows / 16;
        const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvb);
        if (mode == 0) {
            timing_begin("gdn_chain", s);
            gdn_chain_ws_kernel<KD, KS, false><<<grid, 64 * (KS + 4), 0, s>>>(
                q, k, v, h0, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, nvb, scale, out, ht, nullptr);
        } else {
            timing_begin("gdn_summary_chain", s);
            gdn_chain_ws_kernel<KD, KS, true><<<grid, 64 * (KS + 4), 0, s>>>(
                q, k, v, nullptr, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, nvb, scale, nullptr, ht, Mout);
        }
        timing_end(s);
        return hipGetLastError();
    }
    constexpr int NW = 4;
    const int nvb = rows / (16 * NW);
    const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvb);
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

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

// Fragment order of a lower-triangular 64x64 bf16 block M (T or P), as the
// MFMA operand the chain reads it in. Fragment f = FRAG_BASE[ti] + p covers
// rows 16 ti .. 16 ti + 15 and columns 32 p .. 32 p + 31 (p <= ti / 2, the
// blocks right of the diagonal tile being zero); lane (ln, lg) holds 16 bytes:
// M[16 ti + ln][32 p + 4 lg + j] then M[16 ti + ln][32 p + 16 + 4 lg + j],
// j = 0..3. That is the A operand of a 32-deep product reducing over the
// block's columns against a right operand made of two consecutive 16-row
// C tiles, and equally the B operand of the transposed product. Six
// fragments, 6 KB.
constexpr int kTriFrags = 6;
__host__ __device__ constexpr int tri_frag(int ti, int p) { return (ti == 0 ? 0 : ti == 1 ? 1 : ti == 2 ? 2 : 4) + p; }

// Write the six fragments of the row-major staged block m (row stride ld) to g.
__device__ __forceinline__ void store_tri_frags(const bf16_t* m, int ld, bf16_t* g) {
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int p = 0; p <= ti / 2; ++p) {
            const bf16_t* r = m + (16 * ti + ln) * ld + 32 * p + 4 * lg;
            const uint2 lo = *reinterpret_cast<const uint2*>(r), hi = *reinterpret_cast<const uint2*>(r + 16);
            *reinterpret_cast<u128*>(g + (tri_frag(ti, p) * 64 + lane) * 8) = u128{lo.x, lo.y, hi.x, hi.y};
        }
}

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
    constexpr int LO = GC + 8;  // staging tile row stride (bf16)
    __shared__ __align__(16) float sA[tri_off(GC)];
    __shared__ __align__(16) bf16_t sO[GC * LO];
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
        for (int i = 0; i < GC * LO / 8 / 64; ++i) *reinterpret_cast<u128*>(sO + 8 * (lane + 64 * i)) = u128{0u, 0u, 0u, 0u};
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
                if (WANT_P && i <= t) sO[t * LO + i] = f2bf(scale * d * pq[r]);
            }
        }
        __syncthreads();
        if constexpr (WANT_P) store_tri_frags(sO, LO, gP);
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
        // stored as T diag(beta): column j scaled by beta_j (zero past the chunk's end)
#pragma unroll
        for (int t = 0; t < GC; ++t) sO[t * LO + lane] = f2bf(x[t] * bv);
        __syncthreads();
        store_tri_frags(sO, LO, gT);
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
// ST + Out, bf16: one workgroup = one 16-row state slice of one chain, four
// wavefronts (one per SIMD).
//
//  - Wavefront 0 runs the state recurrence alone, the slice state held in
//    float32 MFMA accumulators for the whole chain: per chunk X = K S^T,
//    Y = diag(beta) (V - diag(Gamma) X), R = T Y and S <- Gamma_L S + (e R)^T K,
//    with no exchange between wavefronts on that path. The C tile of each
//    product is the operand of the next as it stands (sf_device.h); beta is
//    carried by the stored T (T diag(beta)), so Y = V - diag(Gamma) X here.
//  - Wavefront 3 feeds it: it moves chunk c+3 (K, T, the slice's V, the
//    coefficients) from global memory straight into LDS with 16-byte direct
//    loads (no register staging) while the chain works on chunk c, four
//    chunk buffers deep.
//  - Wavefronts 1 and 2 form chunk c-1's output
//    O^T = scale diag(Gamma) (S Q^T) + R^T P^T, two token tiles each, from
//    the bf16 state and residual fragments wavefront 0 leaves in LDS, with
//    Q and P fetched into registers one chunk ahead, and store it with
//    8-byte row stores.
//  One workgroup barrier per chunk.
//
// State tiles: S[kt], kt = 2p + h, is the C tile of S^T whose row 4 lg + j
// stands for key column k = 32 p + 8 lg + 4 h + j and whose column ln for
// state row row0 + ln. The pairs (S[2p], S[2p+1]) then give lane group lg the
// eight consecutive columns 32 p + 8 lg .. + 7, so K and Q rows enter the
// products as plain 16-byte row loads.
//
// K in LDS: fragment (u, p) (u = token tile, p = 32-column pair) is 1 KB,
// slot 16 lg + (ln ^ 4 lg) holding K[16 u + ln][32 p + 8 lg .. + 7]. Row
// fragments read one slot per lane; the transposed reads that build K^T
// fragments for the state update take 8 bytes from 16 different slots per
// 16 lanes. The XOR swizzle keeps both patterns free of bank conflicts.
// ---------------------------------------------------------------------------
template <int KD, bool SUMMARY>
struct ChainLds {
    static constexpr int KP = KD / 32, KB = KD / 16;
    static constexpr int NBUF = 4;                                   // chunks c .. c+3 resident
    static constexpr int OFF_K = 0;                                  // 4 KP fragments of 1 KB
    static constexpr int OFF_T = OFF_K + 4 * KP * 1024;              // kTriFrags fragments of 1 KB
    static constexpr int OFF_V = OFF_T + kTriFrags * 1024;           // V slice [64][16] bf16
    static constexpr int OFF_C = OFF_V + GC * 16 * 2;                // coefficients float[256]
    static constexpr int BUF = OFF_C + 256 * 4;
    static constexpr int NLOAD = 4 * KP + kTriFrags + 2 + 1;         // direct-load instructions per chunk
    static constexpr int OFF_SF = NBUF * BUF;                        // [2][KB][64] x 8 B  bf16 state
    static constexpr int OFF_RB = OFF_SF + (SUMMARY ? 0 : 2 * KB * 512);  // [2][4][64] x 8 B  bf16 R
    static constexpr int BYTES = OFF_RB + (SUMMARY ? 0 : 2 * 4 * 512);
};

__device__ __forceinline__ int kslot(int ln, int lg) { return 16 * lg + (ln ^ (4 * lg)); }

// 16-byte direct load global -> LDS: lane l's 16 bytes land at dst + 16 l.
__device__ __forceinline__ void load_lds16(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat8(i16x4 x, i16x4 y) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int KD, bool SUMMARY>
__global__ __launch_bounds__(256) void gdn_chain_1w_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const uint8_t* __restrict__ fac, int T, int H, int HK, int V, int n_seq, int nc, int nvb,
    float scale, bf16_t* __restrict__ out, float* __restrict__ ht, float* __restrict__ Mout) {
    typedef ChainLds<KD, SUMMARY> SM;
    typedef Elem<bf16_t> El;
    constexpr int KP = SM::KP, KB = SM::KB;

    __shared__ __align__(16) uint8_t smem[SM::BYTES];

    int chain, vb;
    xcd_split(blockIdx.x, nvb, chain, vb);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, hk = h / (H / HK);
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = 16 * vb;       // first state row of this slice
    const bool vrows = row0 < V;    // value rows (else transition rows, summary only)

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
    auto buf = [&](int c) __attribute__((always_inline)) { return smem + (c % SM::NBUF) * SM::BUF; };
    auto record = [&](int c) __attribute__((always_inline)) {
        return fac + ((size_t)(slot0 + c) * H + h) * rec_bytes;
    };
    // Each role below runs its own loop with exactly one barrier per chunk (plus one before the
    // first chunk), so the roles' registers never overlap; every wavefront's own memory traffic
    // is complete (explicit waits) before it reaches a barrier.
    auto barrier = [] __attribute__((always_inline)) () { asm volatile("s_barrier" ::: "memory"); };

    if (wave == 0) {
        // ================= the state recurrence =================
        f32x4 S[KB];
#pragma unroll
        for (int kt = 0; kt < KB; ++kt) {
            const int kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1), row = row0 + ln;
            if constexpr (!SUMMARY) {
                S[kt] = h0 ? *reinterpret_cast<const f32x4*>(h0 + (((size_t)n * H + h) * V + row) * KD + kk) : zero4();
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[kt][r] = (!vrows && kk + r == row - V) ? 1.f : 0.f;
            }
        }
        // chunk operands, read from LDS one barrier ahead of use
        bf16x8 Kf[4][KP], Tf[kTriFrags];
        f32x4 gam[4], ec[4];
        i16x4 Vf[4];
        float gl;
        auto prefetch = [&](int c) __attribute__((always_inline)) {
            const uint8_t* B = buf(c);
            const float* sC = reinterpret_cast<const float*>(B + SM::OFF_C);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                gam[u] = *reinterpret_cast<const f32x4*>(sC + 16 * u + 4 * lg);
                ec[u] = *reinterpret_cast<const f32x4*>(sC + 64 + 16 * u + 4 * lg);
                Vf[u] = vrows ? frag_rows_t(B + SM::OFF_V, 16, 16 * u, 0) : i16x4{0, 0, 0, 0};
            }
            gl = sC[63];
#pragma unroll
            for (int f = 0; f < kTriFrags; ++f)
                Tf[f] = *reinterpret_cast<const bf16x8*>(B + SM::OFF_T + f * 1024 + lane * 16);
            // K row fragments last: X waits on them first
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int p = 0; p < KP; ++p)
                    Kf[u][p] = *reinterpret_cast<const bf16x8*>(B + SM::OFF_K + (u * KP + p) * 1024 + kslot(ln, lg) * 16);
        };
        barrier();
        if (nch > 0) prefetch(0);
        for (int c = 0; c < nch; ++c) {
            const uint8_t* B = buf(c);
            // bf16 copy of the entry state: B operand of X, and left for the output wavefronts
            i16x4 Sf[KB];
#pragma unroll
            for (int kt = 0; kt < KB; ++kt) Sf[kt] = El::pack(S[kt]);
            // X = K S^T
            f32x4 X[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                X[u] = zero4();
#pragma unroll
                for (int p = 0; p < KP; ++p) X[u] = mma32(Kf[u][p], cat8(Sf[2 * p], Sf[2 * p + 1]), X[u]);
            }
            // K^T fragments for the state update: transposed reads of the swizzled K fragments;
            // lane i of group g points at token 16 u + 4 g + i/4, columns 32 p + 8 (i%4) + 4 h
            i16x4 Ka[KB][4];
            {
                const uint8_t* BK = B + SM::OFF_K;
                typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
                for (int kt = 0; kt < KB; ++kt)
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int p = kt >> 1, hh = kt & 1;
                        const int tl = 4 * lg + (ln >> 2), cl = ln & 3;
                        const uint8_t* ptr = BK + (u * KP + p) * 1024 + kslot(tl, cl) * 16 + 8 * hh;
                        Ka[kt][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(ptr));
                    }
            }
            if constexpr (!SUMMARY) {
                i16x4* sSf = reinterpret_cast<i16x4*>(smem + SM::OFF_SF) + (c & 1) * KB * 64;
#pragma unroll
                for (int kt = 0; kt < KB; ++kt) sSf[kt * 64 + lane] = Sf[kt];
            }
            // Y = V - Gamma X (beta is folded into the stored T)
            i16x4 Yf[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) Yf[u] = El::pack(El::unpack(Vf[u]) - gam[u] * X[u]);
            // R = T diag(beta) Y (T lower triangular, fragment pairs of 32 columns)
            f32x4 R[4];
            const bf16x8 Y01 = cat8(Yf[0], Yf[1]), Y23 = cat8(Yf[2], Yf[3]);
            R[0] = mma32(Tf[tri_frag(0, 0)], Y01, zero4());
            R[1] = mma32(Tf[tri_frag(1, 0)], Y01, zero4());
            R[2] = mma32(Tf[tri_frag(2, 1)], Y23, mma32(Tf[tri_frag(2, 0)], Y01, zero4()));
            R[3] = mma32(Tf[tri_frag(3, 1)], Y23, mma32(Tf[tri_frag(3, 0)], Y01, zero4()));
            i16x4 ER[4];
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) ER[ti] = El::pack(R[ti] * ec[ti]);
            if constexpr (!SUMMARY) {
                i16x4* sRb = reinterpret_cast<i16x4*>(smem + SM::OFF_RB) + (c & 1) * 4 * 64;
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) sRb[ti * 64 + lane] = El::pack(R[ti]);
            }
            // S^T <- Gamma_L S^T + K^T (e R)
            const bf16x8 E01 = cat8(ER[0], ER[1]), E23 = cat8(ER[2], ER[3]);
#pragma unroll
            for (int kt = 0; kt < KB; ++kt) {
                f32x4 acc = S[kt] * gl;
                acc = mma32(cat8(Ka[kt][0], Ka[kt][1]), E01, acc);
                acc = mma32(cat8(Ka[kt][2], Ka[kt][3]), E23, acc);
                S[kt] = acc;
            }
            // this chunk's LDS writes are complete before the barrier; the next chunk's operands
            // (filled before the previous barrier) are read now and land while the barrier is waited on
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (c + 1 < nch) prefetch(c + 1);
            barrier();
        }
#pragma unroll
        for (int kt = 0; kt < KB; ++kt) {
            const int kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1), row = row0 + ln;
            if (vrows) {
                if (ht) *reinterpret_cast<f32x4*>(ht + (((size_t)n * H + h) * V + row) * KD + kk) = S[kt];
            } else if constexpr (SUMMARY) {
                *reinterpret_cast<f32x4*>(Mout + (((size_t)n * H + h) * KD + (row - V)) * KD + kk) = S[kt];
            }
        }
    } else if (wave == 3) {
        // ================= feeder: direct loads, chunk c+3 while the chain is on chunk c =================
        // padded rows of a partial chunk repeat its last token (finite values that the stored
        // T diag(beta) and e = 0 keep out of every result)
        auto feed = [&](int c) __attribute__((always_inline)) {
            const int t0 = bos + c * GC, L = min(GC, eos - t0);
            uint8_t* B = buf(c);
            const uint8_t* rec = record(c);
#pragma unroll
            for (int m = 0; m < SM::NLOAD; ++m) {
                if (m < 4 * KP) {
                    const int u = m / KP, p = m % KP;
                    const int t = min(16 * u + (ln ^ (4 * lg)), L - 1);
                    load_lds16(k + ((size_t)(b * T + t0 + t) * HK + hk) * KD + 32 * p + 8 * lg, B + SM::OFF_K + m * 1024);
                } else if (m < 4 * KP + kTriFrags) {
                    const int f = m - 4 * KP;
                    load_lds16(rec + f * 1024 + lane * 16, B + SM::OFF_T + f * 1024);
                } else if (m < 4 * KP + kTriFrags + 2) {
                    // transition-row slices (summary mode) never read it: they load value rows 0..15
                    // so that every chunk issues the same number of loads
                    const int hv = m - 4 * KP - kTriFrags;
                    const int t = min(32 * hv + (lane >> 1), L - 1);
                    load_lds16(v + ((size_t)(b * T + t0 + t) * H + h) * V + (vrows ? row0 : 0) + 8 * (lane & 1),
                               B + SM::OFF_V + hv * 1024);
                } else {
                    load_lds16(rec + 2 * GC * GC * 2 + lane * 16, B + SM::OFF_C);
                }
            }
        };
        // chunks 0 and 1 must have landed before the first barrier, chunk 2 before the second
        for (int c = 0; c < min(nch, 3); ++c) feed(c);
        if (nch > 2)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(SM::NLOAD) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier();
        for (int c = 0; c < nch; ++c) {
            // this wavefront issues no other vector memory operation, so the count is exact
            if (c + 3 < nch) {
                feed(c + 3);
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(SM::NLOAD) : "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            barrier();
        }
    } else {
        // ================= output: wavefront 1 tiles {0, 3}, wavefront 2 tiles {1, 2} =================
        barrier();
        if constexpr (!SUMMARY) {
            struct OutRegs {
                bf16x8 Qf[2][KP], Pf[2][2];
                float gq[2];
            };
            auto tile_of = [&](int i) __attribute__((always_inline)) { return wave == 1 ? 3 * i : 1 + i; };
            auto fetch_out = [&](int c, OutRegs& R) __attribute__((always_inline)) {  // Q, P, Gamma of chunk c
                const int t0 = bos + c * GC, L = min(GC, eos - t0);
                const uint8_t* rec = record(c);
                const bf16_t* gP = reinterpret_cast<const bf16_t*>(rec + GC * GC * 2);
                const float* gC = reinterpret_cast<const float*>(rec + 2 * GC * GC * 2);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int tt = tile_of(i);
                    const int t = min(16 * tt + ln, L - 1);
#pragma unroll
                    for (int p = 0; p < KP; ++p)
                        R.Qf[i][p] = *reinterpret_cast<const bf16x8*>(q + ((size_t)(b * T + t0 + t) * HK + hk) * KD + 32 * p + 8 * lg);
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        if (p <= tt / 2) R.Pf[i][p] = *reinterpret_cast<const bf16x8*>(gP + (tri_frag(tt, p) * 64 + lane) * 8);
                    R.gq[i] = gC[16 * tt + ln];
                }
            };
            auto emit_out = [&](int c, const OutRegs& R) __attribute__((always_inline)) {  // O of chunk c
                const int t0 = bos + c * GC, L = min(GC, eos - t0);
                const i16x4* sSf = reinterpret_cast<const i16x4*>(smem + SM::OFF_SF) + (c & 1) * KB * 64;
                const i16x4* sRb = reinterpret_cast<const i16x4*>(smem + SM::OFF_RB) + (c & 1) * 4 * 64;
                i16x4 Sf[KB], Rb[4];
#pragma unroll
                for (int kt = 0; kt < KB; ++kt) Sf[kt] = sSf[kt * 64 + lane];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) Rb[ti] = sRb[ti * 64 + lane];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int tt = tile_of(i);
                    f32x4 qs = zero4();
#pragma unroll
                    for (int p = 0; p < KP; ++p) qs = mma32(cat8(Sf[2 * p], Sf[2 * p + 1]), R.Qf[i][p], qs);
                    f32x4 o = qs * (R.gq[i] * scale);
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        if (p <= tt / 2) o = mma32(cat8(Rb[2 * p], Rb[2 * p + 1]), R.Pf[i][p], o);
                    const int t = 16 * tt + ln;
                    if (t < L) {
                        const i16x4 ob = El::pack(o);
                        *reinterpret_cast<i16x4*>(out + ((size_t)(b * T + t0 + t) * H + h) * V + row0 + 4 * lg) = ob;
                    }
                }
            };
            // chunk c: fetch chunk c's Q/P into F, emit chunk c-1 from E (register sets alternate)
            auto step = [&](int c, OutRegs& F, const OutRegs& E) __attribute__((always_inline)) {
                fetch_out(c, F);
                if (c > 0) emit_out(c - 1, E);
                barrier();
            };
            OutRegs RA, RB;
            for (int c = 0; c < nch; c += 2) {
                step(c, RA, RB);
                if (c + 1 < nch) step(c + 1, RB, RA);
            }
            if (nch > 0) emit_out(nch - 1, (nch - 1) & 1 ? RB : RA);
        } else {
            for (int c = 0; c < nch; ++c) barrier();
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
        const int nvb = rows / 16;
        const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvb);
        if (mode == 0) {
            timing_begin("gdn_chain", s);
            gdn_chain_1w_kernel<KD, false><<<grid, 256, 0, s>>>(
                q, k, v, h0, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, nvb, scale, out, ht, nullptr);
        } else {
            timing_begin("gdn_summary_chain", s);
            gdn_chain_1w_kernel<KD, true><<<grid, 256, 0, s>>>(
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

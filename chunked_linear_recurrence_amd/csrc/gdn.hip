// Gated Delta Rule chunk forward for gfx950.
//
// The recurrence (attention-gym "Linear Attention", section "Gated Delta
// Rule") is run chunk by chunk with the Pre / ST / Out split of StateFlow
// (Section 2.2, Eq. (2)). For one chunk of L <= 64 tokens of one (sequence,
// value head), entry state S [V x K], within-chunk cumulative gate G,
// Gamma_t = exp(G_t), e_t = exp(G_L - G_t), D_ti = exp(G_t - G_i) (i <= t):
//
//   Pre (state independent)
//     A = diag(beta) (strictly-lower D o K K^T),  T = (I + A)^-1
//     P = scale (D o Q K^T)   (lower triangle incl. diagonal)
//   ST + Out (serial over chunks)
//     X = K S^T,  Y = diag(beta) (V - diag(Gamma) X),  R = T Y
//     O = scale diag(Gamma) Q S^T + P R
//     S <- Gamma_L S + (diag(e) R)^T K
//
// R is the chunk's corrected values (the residuals of the token rule). The
// masked products are contracted raw and then multiplied by decay factors
// exp(G_t - G_i) with i <= t only, so nothing overflows however negative the
// gates are (the gate has no lower bound). The state is carried in float32
// and fed to the MFMA in the q/k/v element type, as the page allows for the
// chunk-entry state.
//
// Kernels:
//   bf16  gdn_prep_bf16_kernel   Pre into per-chunk records (T diag(beta) and
//                                the coefficients), then one of
//         gdn_chain_slice_kernel       the chain and the output, one workgroup per
//                                16-row state slice, P formed on chip
//                                (launches with at most two slices per CU)
//         gdn_chain_head_kernel  the same per (sequence, head) and group of 4
//                                or 8 slices (larger launches, and the
//                                summary pass)
//   f32   gdn_prep_kernel + gdn_chain_kernel
// The bf16 kernels take every per-chunk step from gdn_steps.h, so a
// sequence's results are the same bits whichever of them runs it.
//
// Summary mode (attention-gym "Context Parallelism", "cuDNN local
// execution"): the chain runs on V + K rows, the first V from a zero state
// with the values, the last K from the identity with the values disabled;
// their exit states are S_ext and the transition M.
#include <type_traits>

#include "gdn_steps.h"

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

// ---------------------------------------------------------------------------
// Pre: per (chunk slot, head) -> T, P, coefficients.
// Record layout: T [64][64] ST | P [64][64] ST | coef float[256]:
//   [0,64) Gamma_t  [64,128) e_t  [128,192) beta_t  [192,256) G_t
// (Gamma_L = Gamma_63: padded tokens of a partial chunk have zero gate)
// ---------------------------------------------------------------------------
// The natural-log gate of token row gi and head h: g as given, or the gate transform of the raw
// projection (attention-gym "Linear Attention", "Gate Transforms"), in float32 with the accurate
// exponential and log1p (Pre reads 64 gates per chunk and head, so their cost does not show).
__device__ __forceinline__ float load_gate(const float* __restrict__ g, const GateSrc& gs, size_t gi, int h) {
    if (gs.raw == nullptr) return g[gi];
    const float x = (gs.raw_bf16 ? bf2f(static_cast<const bf16_t*>(gs.raw)[gi]) : static_cast<const float*>(gs.raw)[gi]) +
                    gs.dt_bias[h];
    const float amp = expf(gs.A_log[h]);
    if (gs.bounded) return gs.lower_bound / (1.f + expf(-amp * x));
    return -amp * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));
}

template <typename ST, int KD>
__global__ __launch_bounds__(256) void gdn_prep_kernel(const ST* __restrict__ q, const ST* __restrict__ k,
                                                       const float* __restrict__ g,
                                                       const float* __restrict__ beta,
                                                       const int2* __restrict__ table,
                                                       const int32_t* __restrict__ cu, int T, int H,
                                                       int HK, int nc, float scale, int want_p,
                                                       uint8_t* __restrict__ fac, GateSrc gs) {
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
        const float gv = tid < L ? load_gate(g, gs, gi, h) : 0.f;
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
// Pre, bf16: one wavefront per (chunk slot, head) writes the chunk's coefficients and T diag(beta) into its
// record (gdn_steps.h: pre_all). Read by both bf16 chain kernels (per-slice and per-head).
// ---------------------------------------------------------------------------
// Pre work units u = slot * H + head (heads fastest) in runs of this many units per XCD. The gates
// and beta are [token][head] rows of H floats, so the heads of a chunk read the same lines: in one
// run they come from that XCD's L2 once (a run of one head's chunks would fetch every line on every
// XCD).
constexpr int kPrepXcdRun = 64;
inline unsigned prep_grid(int H, long n_slots) {
    const long units = (long)H * n_slots;
    return (unsigned)(((units + 8 * kPrepXcdRun - 1) / (8 * kPrepXcdRun)) * (8 * kPrepXcdRun));
}

template <int KD>
__global__ __launch_bounds__(64) void gdn_prep_bf16_kernel(const bf16_t* __restrict__ k, const float* __restrict__ g,
                                                           const float* __restrict__ beta, const int2* __restrict__ table,
                                                           const int32_t* __restrict__ cu, int T, int H, int HK, int nc,
                                                           int n_slots, uint8_t* __restrict__ fac, GateSrc gs) {
    constexpr int KP = KD / 32;
    __shared__ __align__(16) uint8_t sc[kSolveBytes];
    __shared__ __align__(16) float scf[256];
    // blockIdx -> unit u = slot * H + h, in runs of kPrepXcdRun units per XCD (workgroups go round-robin
    // over the 8 XCDs)
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int u = (idx / kPrepXcdRun) * (8 * kPrepXcdRun) + xcd * kPrepXcdRun + idx % kPrepXcdRun;
    if (u >= H * n_slots) return;
    const int slot = u / H, h = u % H;
    const int hk = h / (H / HK);
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    int b, t0, L, ci;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L, ci)) return;
    const size_t gi = (size_t)(b * T + t0 + min(lane, L - 1)) * H + h;
    const float graw = gate_load_raw(g, gs, gi);
    const float braw = beta[gi];
    // K rows of the chunk. Rows past a partial chunk's end repeat its last token: they only reach entries
    // that are never read or are cancelled exactly (rows of A scaled by beta = 0; columns of P that meet
    // padded tokens only, and the zero T diag(beta) columns of padded tokens)
    bf16x8 kf[4][KP];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const int t = 16 * R + ln;
        const bf16_t* row = k + ((size_t)(b * T + t0 + min(t, L - 1)) * HK + hk) * KD + 8 * lg;
#pragma unroll
        for (int p = 0; p < KP; ++p) kf[R][p] = *reinterpret_cast<const bf16x8*>(row + 32 * p);
    }
    const float G = wave_inclusive_scan(lane < L ? gate_finish(graw, gs, gate_head(gs, h)) : 0.f);
    const float bv = lane < L ? braw : 0.f;
    uint8_t* rec = fac + ((size_t)slot * H + h) * kGdnRecordBf16;
    pre_all<KP>(kf, G, bv, (lds_f32*)scf, reinterpret_cast<float*>(rec + kRecCoefOffset), (lds_u8*)sc, rec);
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
// ST + Out, bf16, one workgroup per (sequence, head) and group of 16-row slices (the output pass's
// 8 value slices; the summary pass's 16, value and transition rows), for launches with more slices
// than the GPU holds at once. There every CU runs workgroup after workgroup, and the chunk's shared
// operands (K and Q rows, T, coefficients) are loaded once per group rather than once per slice.
// Pre (gdn_prep_bf16_kernel) has written T diag(beta) and the coefficients of every chunk.
//  - Wavefronts 0..7 each run SPW slices' whole chunk step (one in the output pass, two in the
//    summary pass) with the states in registers: X = K S^T, Y = V - Gamma X, R = T diag(beta) Y,
//    O = scale Gamma Q S^T + P R, S <- Gamma_L S + K^T (e R). The output pass takes each slice's
//    step from gdn_steps.h (SliceOps), as the per-slice kernel does.
//  - Wavefronts 8 and 9 move chunk c+1 (K and Q rows, T, coefficients, the eight V slices) into
//    the other of two LDS buffers with 16-byte direct loads while chunk c computes and, in the
//    summary pass, touch the lines of chunk c+2 so that those loads find them in L2.
//  - Wavefront 10 (output pass only) forms P_c = scale (D o Q_c K_c^T) from the K and Q rows in
//    LDS (gdn_steps.h form_p) while the slice wavefronts form X, Y and R, once for the eight slices.
// One workgroup barrier per chunk (two in the output pass: P_c is complete before the outputs).
// ---------------------------------------------------------------------------
template <int KD, bool SUMMARY, int NCW_ = 8>
struct HeadLds {
    typedef RowBlock<KD> RBk;
    static constexpr int KP = KD / 32, KB = KD / 16;
    static constexpr int SPW = SUMMARY ? 2 : 1;                        // slices per slice wavefront
    static constexpr int NCW = SUMMARY ? 8 : NCW_;                     // slice wavefronts
    static constexpr int NPW = SUMMARY ? 0 : 2;                        // wavefronts forming P
    static constexpr int NS = NCW * SPW;                               // slices per workgroup
    static constexpr int NVS = SUMMARY ? 8 : NS;                       // V slices held (V <= 128)
    static constexpr int THREADS = 64 * (NCW + 2 + NPW);
    static constexpr int OFF_K = 0;                                    // K rows (RowBlock)
    static constexpr int OFF_Q = OFF_K + RBk::BYTES;                   // Q rows (RowBlock)
    static constexpr int OFF_T = OFF_Q + (SUMMARY ? 0 : RBk::BYTES);   // kTriFrags fragments of 1 KB
    static constexpr int OFF_P = OFF_T + kTriFrags * 1024;             // kTriFrags fragments of 1 KB
    static constexpr int OFF_C = OFF_P + (SUMMARY ? 0 : kTriFrags * 1024);  // coefficients float[256]
    static constexpr int OFF_V = OFF_C + 256 * 4;                      // [NVS][64][16] bf16 V slices
    static constexpr int BUF = OFF_V + NVS * GC * 16 * 2;
    static constexpr int OFF_JUNK = 2 * BUF;                           // sink of cache warm-up loads
    static constexpr int BYTES = OFF_JUNK + 128 * 4;
    static_assert(BYTES <= 160 * 1024, "LDS plan exceeds the CU's 160 KB");
};

template <int KD, bool SUMMARY, int NCW_>
__global__ __launch_bounds__((HeadLds<KD, SUMMARY, NCW_>::THREADS)) void gdn_chain_head_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const uint8_t* __restrict__ fac, int T, int H, int HK, int V, int n_seq, int nc, int ngrp,
    float scale, bf16_t* __restrict__ out, float* __restrict__ ht, float* __restrict__ Mout) {
    typedef HeadLds<KD, SUMMARY, NCW_> SM;
    typedef RowBlock<KD> RBk;
    typedef Elem<bf16_t> El;
    constexpr int KP = SM::KP, KB = SM::KB, NS = SM::NS, SPW = SM::SPW, NCW = SM::NCW;
    constexpr int UST = (16 / RBk::RPB) * 1024;  // byte step of one 16-row token tile in a row block

    __shared__ __align__(16) uint8_t smem[SM::BYTES];
    lds_u8* const lds0 = (lds_u8*)smem;

    int chain, grp;
    xcd_split(blockIdx.x, ngrp, chain, grp);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, hk = h / (H / HK);
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rows = SUMMARY ? V + KD : V;

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
    const size_t rec_bytes = kGdnRecordBf16;
    auto buf = [&](int c) __attribute__((always_inline)) { return lds0 + (c & 1) * SM::BUF; };
    auto record = [&](int c) __attribute__((always_inline)) {
        return fac + ((size_t)(slot0 + c) * H + h) * rec_bytes;
    };
    auto barrier = [] __attribute__((always_inline)) () { asm volatile("s_barrier" ::: "memory"); };

    if (wave < NCW) {
        // ================= SPW slices: the state recurrence and the output =================
        // rows is a multiple of 16 SPW, so the wavefront's slices are all active or all not, and all
        // value rows or all transition rows
        const int row0 = 16 * (grp * NS + SPW * wave);
        const bool active = row0 < rows;
        const bool vrows = row0 < V;  // value rows (else transition rows, summary only)
        const uint32_t vmask = vrows ? 0xffffffffu : 0u;
        f32x4 S[SPW][KB];
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
            for (int kt = 0; kt < KB; ++kt) {
                const int kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1), row = row0 + 16 * sl + ln;
                if constexpr (!SUMMARY) {
                    S[sl][kt] = (active && h0) ? *reinterpret_cast<const f32x4*>(h0 + (((size_t)n * H + h) * V + row) * KD + kk) : zero4();
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) S[sl][kt][r] = (!vrows && kk + r == row - V) ? 1.f : 0.f;
                }
            }
        int orow[KP], otr[KP];
#pragma unroll
        for (int p = 0; p < KP; ++p) {
            orow[p] = RBk::off(ln, 4 * p + lg);                             // row fragment (0, p)
            otr[p] = RBk::off(4 * lg + (ln >> 2), 4 * p + (ln & 3));        // transposed read, column pair p
        }
        // V slice (row0 / 16 + sl) read transposed; transition rows read slice 0 and mask it
        const int off_v = SM::OFF_V + ((vrows ? row0 - 16 * grp * NS : 0) * GC + (4 * lg + (ln >> 2)) * 16 + 4 * (ln & 3)) * 2;
        barrier();
        // Output rows of a step are held in registers and stored at the start of the next step,
        // after its barrier: stores issued in the middle of a step compete with that step's
        // global-to-LDS fill.
        i16x4 po[4][SPW];
        bf16_t* pa[4];
        bool pv[4] = {false, false, false, false};
        auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                if (pv[tt])
#pragma unroll
                    for (int sl = 0; sl < SPW; ++sl) *reinterpret_cast<i16x4*>(pa[tt] + 16 * sl) = po[tt][sl];
        };
        for (int c = 0; c < nch; ++c) {
            if constexpr (!SUMMARY) if (active) flush();
            if (active) {
                lds_u8* B = buf(c);
                lds_u8* KR = B + SM::OFF_K;
                const lds_f32* cf = (const lds_f32*)(B + SM::OFF_C);
                if constexpr (!SUMMARY) {
                    // one slice: the chunk step of gdn_steps.h
                    typedef SliceOps<KD> Ops;
                    i16x4 Sf[KB];
#pragma unroll
                    for (int kt = 0; kt < KB; ++kt) Sf[kt] = El::pack(S[0][kt]);
                    f32x4 R[4];
                    i16x4 ER[4];
                    Ops::residual(Sf, KR, B + off_v, vmask, cf, B + SM::OFF_T, R, ER);
                    barrier();  // P_c complete (the P wavefronts)
                    const int t0 = bos + c * GC, L = min(GC, eos - t0);
                    i16x4 Rb[4];
#pragma unroll
                    for (int ti = 0; ti < 4; ++ti) Rb[ti] = El::pack(R[ti]);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        bf16x8 qf[KP], pf[2];
#pragma unroll
                        for (int p = 0; p < KP; ++p) qf[p] = *(lds_bf16x8*)(B + SM::OFF_Q + orow[p] + tt * UST);
#pragma unroll
                        for (int pp = 0; pp < 2; ++pp)
                            pf[pp] = pp <= tt / 2 ? *(lds_bf16x8*)(B + SM::OFF_P + tri_frag(tt, pp) * 1024 + lane * 16) : bf16x8{};
                        const float gq = cf[16 * tt + ln] * scale;
                        const f32x4 o = Ops::out_tile(tt, Sf, Rb, qf, gq, pf);
                        const int t = 16 * tt + ln;
                        pa[tt] = out + ((size_t)(b * T + t0 + t) * H + h) * V + row0 + 4 * lg;
                        pv[tt] = t < L;
                        po[tt][0] = El::pack(o);
                    }
                    Ops::update(S[0], ER, KR, cf[63]);
                } else {
                    // bf16 entry states: B operands of X and A operands of the output
                    i16x4 Sf[SPW][KB];
    #pragma unroll
                    for (int sl = 0; sl < SPW; ++sl)
    #pragma unroll
                        for (int kt = 0; kt < KB; ++kt) Sf[sl][kt] = El::pack(S[sl][kt]);
                    // X = K S^T
                    f32x4 X[SPW][4];
    #pragma unroll
                    for (int u = 0; u < 4; ++u) {
    #pragma unroll
                        for (int sl = 0; sl < SPW; ++sl) X[sl][u] = zero4();
    #pragma unroll
                        for (int p = 0; p < KP; ++p) {
                            const bf16x8 kr = *(lds_bf16x8*)(KR + orow[p] + u * UST);
    #pragma unroll
                            for (int sl = 0; sl < SPW; ++sl) X[sl][u] = mma32(kr, cat8(Sf[sl][2 * p], Sf[sl][2 * p + 1]), X[sl][u]);
                        }
                    }
                    // Y = V - Gamma X (beta is folded into T)
                    i16x4 Yf[SPW][4];
    #pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const f32x4 gam = *(const lds_f32x4*)(cf + 16 * u + 4 * lg);
    #pragma unroll
                        for (int sl = 0; sl < SPW; ++sl) {
                            const i16x4 vx = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(B + off_v + sl * GC * 16 * 2 + 16 * u * 16 * 2));
                            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                            const i16x4 Vf = __builtin_bit_cast(i16x4, __builtin_bit_cast(u32x2, vx) & vmask);
                            Yf[sl][u] = El::pack(El::unpack(Vf) - gam * X[sl][u]);
                        }
                    }
                    // R = T diag(beta) Y (T lower triangular, fragment pairs of 32 columns)
                    bf16x8 Tf[kTriFrags];
    #pragma unroll
                    for (int f = 0; f < kTriFrags; ++f) Tf[f] = *(lds_bf16x8*)(B + SM::OFF_T + f * 1024 + lane * 16);
                    f32x4 R[SPW][4];
    #pragma unroll
                    for (int sl = 0; sl < SPW; ++sl) {
                        const bf16x8 Y01 = cat8(Yf[sl][0], Yf[sl][1]), Y23 = cat8(Yf[sl][2], Yf[sl][3]);
                        R[sl][0] = mma32(Tf[tri_frag(0, 0)], Y01, zero4());
                        R[sl][1] = mma32(Tf[tri_frag(1, 0)], Y01, zero4());
                        R[sl][2] = mma32(Tf[tri_frag(2, 1)], Y23, mma32(Tf[tri_frag(2, 0)], Y01, zero4()));
                        R[sl][3] = mma32(Tf[tri_frag(3, 1)], Y23, mma32(Tf[tri_frag(3, 0)], Y01, zero4()));
                    }
                    i16x4 ER[SPW][4];
    #pragma unroll
                    for (int ti = 0; ti < 4; ++ti) {
                        const f32x4 ec = *(const lds_f32x4*)(cf + 64 + 16 * ti + 4 * lg);
    #pragma unroll
                        for (int sl = 0; sl < SPW; ++sl) ER[sl][ti] = El::pack(R[sl][ti] * ec);
                    }
                    // S^T <- Gamma_L S^T + K^T (e R)
                    const float gl = cf[63];
                    bf16x8 E01[SPW], E23[SPW];
    #pragma unroll
                    for (int sl = 0; sl < SPW; ++sl) {
                        E01[sl] = cat8(ER[sl][0], ER[sl][1]);
                        E23[sl] = cat8(ER[sl][2], ER[sl][3]);
                    }
    #pragma unroll
                    for (int kt = 0; kt < KB; ++kt) {
                        const int p = kt >> 1, hh = kt & 1;
                        i16x4 Ka[4];
    #pragma unroll
                        for (int u = 0; u < 4; ++u)
                            Ka[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(KR + otr[p] + 8 * hh + u * UST));
                        const bf16x8 K01 = cat8(Ka[0], Ka[1]), K23 = cat8(Ka[2], Ka[3]);
    #pragma unroll
                        for (int sl = 0; sl < SPW; ++sl) {
                            f32x4 acc = S[sl][kt] * gl;
                            acc = mma32(K01, E01[sl], acc);
                            acc = mma32(K23, E23[sl], acc);
                            S[sl][kt] = acc;
                        }
                    }
                }
            } else {
                if constexpr (!SUMMARY) barrier();  // the P_c barrier of the active slices
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            barrier();
        }
        if constexpr (!SUMMARY) if (active) flush();
        if (active) {
#pragma unroll
            for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
                for (int kt = 0; kt < KB; ++kt) {
                    const int kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1), row = row0 + 16 * sl + ln;
                    if (vrows) {
                        if (ht) *reinterpret_cast<f32x4*>(ht + (((size_t)n * H + h) * V + row) * KD + kk) = S[sl][kt];
                    } else if constexpr (SUMMARY) {
                        *reinterpret_cast<f32x4*>(Mout + (((size_t)n * H + h) * KD + (row - V)) * KD + kk) = S[sl][kt];
                    }
                }
        }
    } else if (wave < NCW + 2) {
        // ================= feeders: direct loads into LDS, two wavefronts =================
        // wavefront 8: K rows, T, coefficients, V slices 0..3; wavefront 9: Q rows, V slices 4..7.
        // Rows past the end of a partial chunk repeat its last token (finite values that the
        // stored T diag(beta) and e = 0 keep out of the state, and whose outputs are not stored).
        const int fi = wave - NCW;
        const size_t krs = (size_t)HK * KD * 2, vrs = (size_t)H * V * 2;  // token strides (bytes)
        auto feed_rows = [&](const bf16_t* src, int c, lds_u8* dst) __attribute__((always_inline)) {
            const int t0 = bos + c * GC, L = min(GC, eos - t0);
            const uint8_t* base = reinterpret_cast<const uint8_t*>(src + ((size_t)(b * T + t0) * HK + hk) * KD);
#pragma unroll
            for (int m = 0; m < RBk::NLOAD; ++m) {
                const int r = m * RBk::RPB + lane / RBk::PCS, pc = lane % RBk::PCS;
                load_lds16(base + (size_t)min(r, L - 1) * krs + 16 * (pc ^ RBk::swz(r)), (uint8_t*)(dst + m * 1024));
            }
        };
        // V slice j [64][16]: instruction hv, lane l -> token 32 hv + l/2, values 16 j + 8 (l%2) .. + 7
        auto feed_v = [&](int c, int j) __attribute__((always_inline)) {
            const int t0 = bos + c * GC, L = min(GC, eos - t0);
            const uint8_t* vb0 = reinterpret_cast<const uint8_t*>(v + (size_t)(b * T + t0) * H * V + (size_t)h * V);
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                const int t = min(32 * hv + (lane >> 1), L - 1);
                load_lds16(vb0 + (size_t)t * vrs + (16 * (grp * NS + j) + 8 * (lane & 1)) * 2,
                           (uint8_t*)(buf(c) + SM::OFF_V + j * GC * 16 * 2 + hv * 1024));
            }
        };
        // the V slices this group holds (summary transition rows have none)
        const int vslices = max(0, min(SM::NVS, V / 16 - grp * NS));
        auto issue = [&](int c) __attribute__((always_inline)) {  // returns load instructions issued
            lds_u8* B = buf(c);
            const uint8_t* rec = record(c) + lane * 16;
            int nl = 0;
            if (fi == 0) {
                feed_rows(k, c, B + SM::OFF_K);
#pragma unroll
                for (int f = 0; f < kTriFrags; ++f) load_lds16(rec + f * 1024, (uint8_t*)(B + SM::OFF_T + f * 1024));
                load_lds16(rec + kRecCoefOffset, (uint8_t*)(B + SM::OFF_C));
                nl = RBk::NLOAD + kTriFrags + 1;
                for (int j = 0; j < min(vslices, SM::NVS / 2); ++j) {
                    feed_v(c, j);
                    nl += 2;
                }
            } else {
                if constexpr (!SUMMARY) {
                    feed_rows(q, c, B + SM::OFF_Q);
                    nl = RBk::NLOAD;
                }
                for (int j = SM::NVS / 2; j < vslices; ++j) {
                    feed_v(c, j);
                    nl += 2;
                }
            }
            return nl;
        };
        // Cache warm-up: one 4-byte load per 128-byte line of chunk c, from the list K rows [0, 128),
        // Q rows [128, 256) (K again in summary mode), the head's V rows [256, 384) (two lines per
        // token each), then the record's T [384, 432) and coefficient [432, 440) lines; lane l of
        // wavefront fi touches lines 4 (64 fi + l) .. + 3 (past the end: the last line).
        constexpr int NLINES = 440;
        auto warm = [&](int c) __attribute__((always_inline)) {
            const int t0 = bos + c * GC, L = min(GC, eos - t0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int li = min(4 * (64 * fi + lane) + e, NLINES - 1);
                const uint8_t* a;
                if (li < 256) {
                    const int t = min((li & 127) >> 1, L - 1);
                    const bf16_t* base = (li < 128 || SUMMARY) ? k : q;
                    a = reinterpret_cast<const uint8_t*>(base + ((size_t)(b * T + t0 + t) * HK + hk) * KD) + (li & 1) * (KD >= 128 ? 128 : 0);
                } else if (li < 384) {
                    const int t = min((li - 256) >> 1, L - 1);
                    a = reinterpret_cast<const uint8_t*>(v + ((size_t)(b * T + t0 + t) * H + h) * V) + (li & 1) * (V >= 128 ? 128 : 0);
                } else {
                    const int r = li - 384;
                    const size_t off = r < 48 ? (size_t)r * 128 : (size_t)kRecCoefOffset + (r - 48) * 128;
                    a = record(c) + off;
                }
                __builtin_amdgcn_global_load_lds(a, (__attribute__((address_space(3))) void*)(smem + SM::OFF_JUNK + fi * 256), 4, 0, 0);
            }
        };
        // (loads complete in issue order: the wait after a step's loads and its warm-up leaves only
        // the warm-up in flight)
        // The warm-up runs in summary mode only: in the output pass (Q and V rows as well, 32
        // workgroups per XCD) the touched lines are evicted before their loads come, and on a
        // long input the pass fetched 15 % more than it reads.
        if (nch > 0) issue(0);
        if constexpr (SUMMARY) if (nch > 1) warm(1);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) {
                issue(c + 1);
                if constexpr (SUMMARY) if (c + 2 < nch) warm(c + 2);
            }
            if constexpr (!SUMMARY) barrier();  // the P_c barrier
            if (c + 1 < nch) {
                if (SUMMARY && c + 2 < nch)
                    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            barrier();
        }
    } else {
        // ================= P_c for the output pass: two wavefronts, block rows {0, 3} and {1, 2} =================
        // P^T tiles with K rows as A (rows s) and Q rows as B (columns t): the C tile holds, for lane
        // (ln, lg), P[16 ti + ln][16 tj + 4 lg + r], which is fragment (ti, tj / 2)'s lane content
        // (first or second half), the B operand that pairs with the R fragments of the same tokens.
        // The cumulative gates G are the coefficient block's last quarter.
        if constexpr (!SUMMARY) {
            barrier();
            for (int c = 0; c < nch; ++c) {
                lds_u8* B = buf(c);
                if (wave == NCW + 2)
                    form_p<KD, 0x9>(B + SM::OFF_K, B + SM::OFF_Q, (const lds_f32*)(B + SM::OFF_C), scale, B + SM::OFF_P);
                else
                    form_p<KD, 0x6>(B + SM::OFF_K, B + SM::OFF_Q, (const lds_f32*)(B + SM::OFF_C), scale, B + SM::OFF_P);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                barrier();  // P_c complete
                barrier();  // end of the step
            }
        }
    }
}


// ---------------------------------------------------------------------------
// The bf16 chunk forward chain in one kernel, after Pre: one workgroup per 16-row state slice of a (sequence,
// head) chain, for launches with at most two slices per CU. Pre (gdn_prep_bf16_kernel) has written every
// chunk's T diag(beta) and coefficients; the workgroup streams them with the chunk's K, Q and V rows into LDS
// rings, two chunks ahead of the step that uses them, and forms P itself.
// Eight wavefronts with fixed roles, one workgroup barrier per step; in step s:
//   0     chain:     the slice's float32 state in registers and the whole step of chunk s: X = K S^T from the
//                    bf16 entry state, Y = V - Gamma X, R = T diag(beta) Y, e R and S <- Gamma_L S + K_s^T (e R),
//                    each product's C tile the next one's B operand; the K^T reads of the update are issued
//                    behind the residual's own reads; R of chunk s and the bf16 entry state of chunk s+1 go to
//                    LDS for the output wavefronts
//   1, 2  output:    O of chunk s-1 for token tiles {0, 3} / {1, 2} (its Q rows and Gamma were read into
//                    registers in step s-1, its entry state, R and P come from LDS); then reads chunk s's
//   3, 5  P:         P = scale (D o Q K^T) of chunk s, block rows {0, 3} / {1, 2}
//   4     records:   T diag(beta) and the coefficients of chunk s+2
//   6     feeder:    K rows of chunk s+2 (16-byte direct loads into LDS)
//   7     feeder:    Q rows and the V slice of chunk s+2
// The loading wavefronts wait, before the barrier of step s, only for the loads they issued in step s-1, so
// that a load has a whole step to land. Wavefront w runs on SIMD w % 4: the chain wavefront shares its SIMD
// only with the record loader. Every per-chunk product comes from gdn_steps.h, as in Pre and the per-head
// kernel.
// ---------------------------------------------------------------------------
template <int KD>
struct SliceLds {
    typedef RowBlock<KD> RBk;
    static constexpr int KB = KD / 16;
    static constexpr int RBB = RBk::BYTES;                       // one chunk of K or Q rows
    static constexpr int OFF_K = 0;                              // K rows, ring of 3 chunks
    static constexpr int OFF_Q = OFF_K + 3 * RBB;                // Q rows, ring of 3
    static constexpr int OFF_V = OFF_Q + 3 * RBB;                // the slice's V [64][16] bf16, ring of 3
    static constexpr int OFF_C = OFF_V + 3 * 2048;               // coefficients float[256], ring of 3
    static constexpr int OFF_T = OFF_C + 3 * 1024;               // T diag(beta) fragments, ring of 3
    static constexpr int OFF_P = OFF_T + 3 * kTriFrags * 1024;   // P fragments, ring of 2
    static constexpr int OFF_SF = OFF_P + 2 * kTriFrags * 1024;  // bf16 entry state [KB][64 lanes] x 8 B, ring of 3
    static constexpr int OFF_R = OFF_SF + 3 * KB * 512;          // bf16 R [4][64 lanes] x 8 B, ring of 2
    static constexpr int BYTES = OFF_R + 2 * 2048;
    static_assert(BYTES <= 160 * 1024, "LDS plan exceeds the CU's 160 KB");
};

template <int KD>
__global__ __launch_bounds__(512) void gdn_chain_slice_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const uint8_t* __restrict__ fac, int nc, int T, int H, int HK, int V, int n_seq, int nvb, float scale,
    bf16_t* __restrict__ out, float* __restrict__ ht) {
    typedef SliceLds<KD> SM;
    typedef RowBlock<KD> RBk;
    typedef SliceOps<KD> Ops;
    typedef Elem<bf16_t> El;
    constexpr int KP = KD / 32, KB = KD / 16;
    constexpr int UST = Ops::UST;

    __shared__ __align__(16) uint8_t smem[SM::BYTES];
    lds_u8* const lds0 = (lds_u8*)smem;

    int chain, vb;
    xcd_split(blockIdx.x, nvb, chain, vb);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, hk = h / (H / HK);
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int row0 = 16 * vb;  // first state row of this slice

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
    // ring buffers (chunk index c >= 0)
    auto kbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_K + (c % 3) * SM::RBB; };
    auto qbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_Q + (c % 3) * SM::RBB; };
    auto vbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_V + (c % 3) * 2048; };
    auto cbuf = [&](int c) __attribute__((always_inline)) { return (lds_f32*)(lds0 + SM::OFF_C + (c % 3) * 1024); };
    auto tbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_T + (c % 3) * kTriFrags * 1024; };
    auto pbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_P + (c & 1) * kTriFrags * 1024; };
    auto sfbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_SF + (c % 3) * KB * 512; };
    auto rbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_R + (c & 1) * 2048; };
    auto chunk_len = [&](int c) __attribute__((always_inline)) { return min(GC, eos - (bos + c * GC)); };
    auto barrier = [] __attribute__((always_inline)) () { asm volatile("s_barrier" ::: "memory"); };
    // Every wavefront passes one barrier before the steps and one at the end of each step s = -2 .. nch.

    if (wave == 0) {
        // ================= chain: the slice's float32 state and the whole chunk step =================
        __builtin_amdgcn_s_setprio(2);  // the chain is the critical path: first pick of its SIMD
        const int off_v = ((4 * lg + (ln >> 2)) * 16 + 4 * (ln & 3)) * 2;  // transposed V reads
        f32x4 S[KB];
        i16x4 Sf[KB];
#pragma unroll
        for (int kt = 0; kt < KB; ++kt) {
            const int kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1), row = row0 + ln;
            S[kt] = h0 ? *reinterpret_cast<const f32x4*>(h0 + (((size_t)n * H + h) * V + row) * KD + kk) : zero4();
            Sf[kt] = El::pack(S[kt]);
        }
        auto put_state = [&](int c) __attribute__((always_inline)) {  // bf16 entry state of chunk c
#pragma unroll
            for (int kt = 0; kt < KB; ++kt) *(lds_i16x4*)(sfbuf(c) + kt * 512 + lane * 8) = Sf[kt];
        };
        if (nch > 0) put_state(0);
        wave_lds_sync();
        barrier();
        for (int s = -2; s <= nch; ++s) {
            if (s >= 0 && s < nch) {
                // Gamma_L is read ahead of everything; the K^T fragments of the update are read while the residual
                // computes, half of the key tiles after X (with Gamma_L S formed then) and half after Y
                i16x4 Ka[KB / 2][4], Kb[KB / 2][4];
                f32x4 R[4];
                i16x4 ER[4];
                float gl;
                Ops::residual_split(Sf, kbuf(s), vbuf(s) + off_v, 0xffffffffu, cbuf(s), tbuf(s), R, ER,
                                    [&]() __attribute__((always_inline)) { gl = cbuf(s)[63]; },
                                    [&]() __attribute__((always_inline)) {
                                        Ops::template read_kt<0, KB / 2>(kbuf(s), Ka);
#pragma unroll
                                        for (int kt = 0; kt < KB; ++kt) S[kt] = S[kt] * gl;
                                    },
                                    [&]() __attribute__((always_inline)) { Ops::template read_kt<KB / 2, KB / 2>(kbuf(s), Kb); });
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) *(lds_i16x4*)(rbuf(s) + ti * 512 + lane * 8) = El::pack(R[ti]);
                Ops::template update_halves<KB>(S, ER, Ka, Kb, 1.f);  // S holds Gamma_L S already
#pragma unroll
                for (int kt = 0; kt < KB; ++kt) Sf[kt] = El::pack(S[kt]);
                // R of chunk s and the entry state of chunk s (written in step s - 1) are in LDS; the entry state
                // of chunk s + 1 is written now and waited for at the end of the next step
                wave_lds_sync();
                if (s + 1 < nch) put_state(s + 1);
            }
            barrier();
        }
        if (ht) {
#pragma unroll
            for (int kt = 0; kt < KB; ++kt) {
                const int kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1), row = row0 + ln;
                *reinterpret_cast<f32x4*>(ht + (((size_t)n * H + h) * V + row) * KD + kk) = S[kt];
            }
        }
    } else if (wave <= 2) {
        // ================= output: wavefront 1 token tiles {0, 3}, wavefront 2 tiles {1, 2} =================
        auto tile_of = [&](int i) __attribute__((always_inline)) { return wave == 1 ? 3 * i : 1 + i; };
        bf16x8 Qf[2][KP];
        float gq[2];
        barrier();
        for (int s = -2; s <= nch; ++s) {
            const int c = s - 1;  // chunk whose output is formed now
            if (c >= 0 && c < nch) {
                const int t0 = bos + c * GC, L = chunk_len(c);
                i16x4 Rb[4], Sf[KB];
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) Rb[ti] = *(const lds_i16x4*)(rbuf(c) + ti * 512 + lane * 8);
#pragma unroll
                for (int kt = 0; kt < KB; ++kt) Sf[kt] = *(const lds_i16x4*)(sfbuf(c) + kt * 512 + lane * 8);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int tt = tile_of(i);
                    bf16x8 pf[2];
#pragma unroll
                    for (int pp = 0; pp < 2; ++pp)
                        pf[pp] = pp <= tt / 2 ? *(const lds_bf16x8*)(pbuf(c) + tri_frag(tt, pp) * 1024 + lane * 16) : bf16x8{};
                    const f32x4 o = Ops::out_tile(tt, Sf, Rb, Qf[i], gq[i], pf);
                    const int t = 16 * tt + ln;
                    if (t < L) *reinterpret_cast<i16x4*>(out + ((size_t)(b * T + t0 + t) * H + h) * V + row0 + 4 * lg) = El::pack(o);
                }
            }
            if (s >= 0 && s < nch) {
                // chunk s's Q row fragments of the own tiles and scale Gamma of the lane's token (the Q ring
                // slot is refilled in step s + 1)
                const lds_f32* cf = cbuf(s);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int tt = tile_of(i);
#pragma unroll
                    for (int p = 0; p < KP; ++p) Qf[i][p] = *(const lds_bf16x8*)(qbuf(s) + Ops::orow(p) + tt * UST);
                    gq[i] = cf[16 * tt + ln] * scale;
                }
            }
            wave_lds_sync();
            barrier();
        }
    } else if (wave == 3 || wave == 5) {
        // ================= P of chunk s: wavefront 3 block rows {0, 3}, wavefront 5 rows {1, 2} =================
        barrier();
        for (int s = -2; s <= nch; ++s) {
            if (s >= 0 && s < nch) {
                if (wave == 3)
                    form_p<KD, 0x9>(kbuf(s), qbuf(s), cbuf(s), scale, pbuf(s));
                else
                    form_p<KD, 0x6>(kbuf(s), qbuf(s), cbuf(s), scale, pbuf(s));
                wave_lds_sync();
            }
            barrier();
        }
    } else {
        // ================= loaders of chunk s+2: wavefront 4 the records, 6 the K rows, 7 the Q rows and V slice =================
        // Rows past the end of a partial chunk repeat its last token (finite values that the zero beta,
        // T diag(beta) columns and e of padded tokens keep out of every stored result).
        const size_t krs = (size_t)HK * KD * 2, vrs = (size_t)H * V * 2;  // token strides (bytes)
        auto feed_rows = [&](const bf16_t* src, int c, lds_u8* dst) __attribute__((always_inline)) {
            const int L = chunk_len(c);
            const uint8_t* base = reinterpret_cast<const uint8_t*>(src + ((size_t)(b * T + bos + c * GC) * HK + hk) * KD);
#pragma unroll
            for (int m = 0; m < RBk::NLOAD; ++m) {
                const int r = m * RBk::RPB + lane / RBk::PCS, pc = lane % RBk::PCS;
                load_lds16(base + (size_t)min(r, L - 1) * krs + 16 * (pc ^ RBk::swz(r)), (uint8_t*)(dst + m * 1024));
            }
        };
        // V slice [64][16]: instruction hv, lane l -> token 32 hv + l / 2, values row0 + 8 (l % 2) .. + 7
        auto feed_v = [&](int c) __attribute__((always_inline)) {
            const int L = chunk_len(c);
            const uint8_t* vb0 = reinterpret_cast<const uint8_t*>(v + (size_t)(b * T + bos + c * GC) * H * V + (size_t)h * V);
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                const int t = min(32 * hv + (lane >> 1), L - 1);
                load_lds16(vb0 + (size_t)t * vrs + (row0 + 8 * (lane & 1)) * 2, (uint8_t*)(vbuf(c) + hv * 1024));
            }
        };
        auto feed_rec = [&](int c) __attribute__((always_inline)) {
            const uint8_t* rec = fac + ((size_t)(slot0 + c) * H + h) * kGdnRecordBf16 + lane * 16;
#pragma unroll
            for (int f = 0; f < kTriFrags; ++f) load_lds16(rec + f * 1024, (uint8_t*)(tbuf(c) + f * 1024));
            load_lds16(rec + kRecCoefOffset, (uint8_t*)cbuf(c));
        };
        // loads of a chunk per wavefront (the vmcnt below leaves exactly the latest chunk's loads in flight)
        constexpr int NREC = kTriFrags + 1, NK = RBk::NLOAD, NQV = RBk::NLOAD + 2;
        barrier();
        for (int s = -2; s <= nch; ++s) {
            const int c = s + 2;
            const bool more = c < nch;
            if (more) {
                if (wave == 4)
                    feed_rec(c);
                else if (wave == 6)
                    feed_rows(k, c, kbuf(c));
                else {
                    feed_rows(q, c, qbuf(c));
                    feed_v(c);
                }
            }
            // chunk s+1's loads (issued in step s-1) have landed; chunk s+2's stay in flight
            if (!more)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            else if (wave == 4)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NREC) : "memory");
            else if (wave == 6)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NK) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NQV) : "memory");
            barrier();
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

// Compute units of the current device (cached per device).
int device_cus() {
    static int cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// After Pre, the bf16 forward chain runs in the per-slice kernel (one workgroup per 16-row slice) when the
// launch has at most two slices per CU, else in the per-head kernel. Both read the same factor records and
// take every chunk step from the same code (gdn_steps.h), so the choice changes no result bit; it only
// decides which runs faster.
bool gdn_chain_per_slice(long chains, int V) { return chains * (V / 16) <= 2L * device_cus(); }

template <int KD>
static hipError_t run_gdn_bf16(int mode, const bf16_t* q, const bf16_t* k, const bf16_t* v, const float* g,
                               const float* beta, const float* h0, const int32_t* cu, const GdnWorkspace& ws, int N,
                               int B, int T, int H, int HK, int V, float scale, bf16_t* out, float* ht, float* Mout,
                               hipStream_t s, int stages, const GateSrc& gs) {
    const bool packed = cu != nullptr;
    const long slots = gdn_slots(B, T, N, packed);
    const int nc = (T + GC - 1) / GC;
    const int chains = N * H;
    const bool per_slice = mode == 0 && gdn_chain_per_slice(chains, V);
    hipError_t err;
    if (stages & 1) {
        if (packed) {
            err = launch_chunk_table(cu, N, GC, slots, ws.chunk_off, ws.table, s);
            if (err != hipSuccess) return err;
        }
        if (slots > 0) {
            timing_begin("gdn_prep", s);
            gdn_prep_bf16_kernel<KD><<<prep_grid(H, slots), 64, 0, s>>>(k, g, beta, packed ? ws.table : nullptr, cu, T, H,
                                                                     HK, nc, (int)slots, ws.factors, gs);
            timing_end(s);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
    }
    if (!(stages & 2) || chains == 0) return hipSuccess;
    const int nvb = V / 16;
    if (per_slice) {
        const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvb);
        timing_begin("gdn_chain_slice", s);
        gdn_chain_slice_kernel<KD><<<grid, 512, 0, s>>>(q, k, v, h0, cu, ws.chunk_off, ws.factors, nc, T, H, HK, V, N, nvb,
                                                  scale, out, ht);
        timing_end(s);
        return hipGetLastError();
    }
    // slices per workgroup: the summary pass's 16 (all of a head's V + K rows); the output pass's 4 for packed
    // input, whose longest sequences set the time (smaller workgroups step faster), else 8 (one workgroup per
    // head keeps equal-length chains to one pass over the CUs). Every slice runs the same steps either way.
    const int rows = mode == 0 ? V : V + KD;
    const bool four = mode == 0 && cu != nullptr;
    const int ns = mode != 0 ? HeadLds<KD, true>::NS : four ? HeadLds<KD, false, 4>::NS : HeadLds<KD, false, 8>::NS;
    const int ngrp = (rows / 16 + ns - 1) / ns;
    const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * ngrp);
    if (mode == 0) {
        timing_begin("gdn_chain", s);
        if (four)
            gdn_chain_head_kernel<KD, false, 4><<<grid, HeadLds<KD, false, 4>::THREADS, 0, s>>>(
                q, k, v, h0, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, ngrp, scale, out, ht, nullptr);
        else
            gdn_chain_head_kernel<KD, false, 8><<<grid, HeadLds<KD, false, 8>::THREADS, 0, s>>>(
                q, k, v, h0, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, ngrp, scale, out, ht, nullptr);
    } else {
        timing_begin("gdn_summary_chain", s);
        gdn_chain_head_kernel<KD, true, 8><<<grid, HeadLds<KD, true>::THREADS, 0, s>>>(q, k, v, nullptr, cu, ws.chunk_off, ws.factors, T, H, HK,
                                                             V, N, nc, ngrp, scale, nullptr, ht, Mout);
    }
    timing_end(s);
    return hipGetLastError();
}

template <int KD>
static hipError_t run_gdn_f32(int mode, const float* q, const float* k, const float* v, const float* g,
                              const float* beta, const float* h0, const int32_t* cu, const GdnWorkspace& ws, int N,
                              int B, int T, int H, int HK, int V, float scale, float* out, float* ht, float* Mout,
                              hipStream_t s, int stages, const GateSrc& gs) {
    const bool packed = cu != nullptr;
    const long slots = gdn_slots(B, T, N, packed);
    const int nc = (T + GC - 1) / GC;
    hipError_t err;
    if (packed && (stages & 1)) {
        err = launch_chunk_table(cu, N, GC, slots, ws.chunk_off, ws.table, s);
        if (err != hipSuccess) return err;
    }
    if (slots > 0 && (stages & 1)) {
        timing_begin("gdn_prep", s);
        gdn_prep_kernel<float, KD><<<dim3((unsigned)slots, H), 256, 0, s>>>(
            q, k, g, beta, packed ? ws.table : nullptr, cu, T, H, HK, nc, scale, mode == 0 ? 1 : 0, ws.factors, gs);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (!(stages & 2)) return hipSuccess;
    const int rows = mode == 0 ? V : V + KD;
    const int chains = N * H;
    if (chains == 0) return hipSuccess;
    constexpr int NW = 4;
    const int nvb = rows / (16 * NW);
    const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvb);
    if (mode == 0) {
        timing_begin("gdn_chain", s);
        gdn_chain_kernel<float, KD, NW, false><<<grid, 64 * NW, 0, s>>>(
            q, k, v, h0, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, nvb, scale, out, ht, nullptr);
    } else {
        timing_begin("gdn_summary_chain", s);
        gdn_chain_kernel<float, KD, NW, true><<<grid, 64 * NW, 0, s>>>(
            q, k, v, nullptr, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, nvb, scale, nullptr, ht, Mout);
    }
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_gdn(bool bf16, int mode, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const float* h0, const int32_t* cu,
                      const GdnWorkspace& ws, int N, int B, int T, int H, int HK, int K, int V,
                      float scale, void* out, float* ht, float* Mout, hipStream_t s, int stages,
                      const GateSrc* gate_src) {
    const GateSrc gs = gate_src ? *gate_src : GateSrc{nullptr, 0, nullptr, nullptr, 0, 0.f};
    if (bf16) {
        const bf16_t *qq = (const bf16_t*)q, *kk = (const bf16_t*)k, *vv = (const bf16_t*)v;
        if (K == 128) return run_gdn_bf16<128>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (bf16_t*)out, ht, Mout, s, stages, gs);
        return run_gdn_bf16<64>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (bf16_t*)out, ht, Mout, s, stages, gs);
    }
    const float *qq = (const float*)q, *kk = (const float*)k, *vv = (const float*)v;
    if (K == 128) return run_gdn_f32<128>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (float*)out, ht, Mout, s, stages, gs);
    return run_gdn_f32<64>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (float*)out, ht, Mout, s, stages, gs);
}

}  // namespace sf

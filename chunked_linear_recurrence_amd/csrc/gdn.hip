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

// Locate chunk `slot`: batch row, first token, length, index of the chunk in
// its sequence. false past the end.
__device__ __forceinline__ bool chunk_coords(int slot, const int2* table, const int32_t* cu, int T,
                                             int nc, int& b, int& t0, int& L, int& ci) {
    if (table) {
        const int2 e = table[slot];
        if (e.x < 0) return false;
        b = 0;
        t0 = cu[e.x] + GC * e.y;
        L = min(GC, cu[e.x + 1] - t0);
        ci = e.y;
    } else {
        b = slot / nc;
        ci = slot % nc;
        t0 = ci * GC;
        L = min(GC, T - t0);
    }
    return true;
}
__device__ __forceinline__ bool chunk_coords(int slot, const int2* table, const int32_t* cu, int T,
                                             int nc, int& b, int& t0, int& L) {
    int ci;
    return chunk_coords(slot, table, cu, T, nc, b, t0, L, ci);
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
// Pre, bf16: shared pieces of the two kernels below.
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

// Pre work units u = slot * H + head (heads fastest) in runs of this many units per XCD. The gates
// and beta are [token][head] rows of H floats, so the heads of a chunk read the same lines: in one
// run they come from that XCD's L2 once (a run of one head's chunks would fetch every line on every
// XCD). Neighbouring chunks of a head (the key rows W reads) mostly share a run too.
constexpr int kPrepXcdRun = 64;
inline unsigned prep_grid(int H, long n_slots) {
    const long units = (long)H * n_slots;
    return (unsigned)(((units + 8 * kPrepXcdRun - 1) / (8 * kPrepXcdRun)) * (8 * kPrepXcdRun));
}

// ---------------------------------------------------------------------------
// Pre, bf16: one workgroup of two wavefronts per (chunk slot, head); the two never wait for
// each other (each orders its own LDS traffic).
//  - K and Q rows go straight from global memory into 16x16x32 MFMA fragments (lane (n, g)
//    holds row 16R+n, columns 32p+8g..+7).
//  - Wavefront 0: the within-chunk gates and coefficients; A = diag(beta)(strictly lower
//    D o K K^T) in LDS as packed columns (column i holds rows i+1..63, 16-byte aligned);
//    T = (I + A)^-1 by 16x16 blocks; T diag(beta) out through a 64x64 bf16 staging tile that
//    reuses the A area, in fragment order.
//  - Wavefront 1: its own copy of the gates; P^T = scale (D o K Q^T)^T tile by tile, whose C
//    tiles are already the lane contents of P's fragments, so P goes out from registers.
//  - The key-key block W = K_c K_{c-1}^T from the previous chunk's rows, when a chain kernel that
//    reads it runs on these records (want_w): each wavefront forms half of its fragments
//    (wavefront 0 before its solve, wavefront 1 after P).
//  With one wavefront (NW = 1, for launches larger than the GPU holds at once) the two parts run
//  one after the other.
// ---------------------------------------------------------------------------
template <int KD, bool WANT_P, int NW>
__global__ __launch_bounds__(64 * NW, NW == 2 ? 4 : 1) void gdn_prep_wave_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ beta,
                                                            const int2* __restrict__ table,
                                                            const int32_t* __restrict__ cu, int T, int H,
                                                            int HK, int nc, int n_slots, float scale,
                                                            uint8_t* __restrict__ fac, int want_w, GateSrc gs) {
    constexpr int KP = KD / 32;
    static_assert(tri_off(GC) * 4 >= GC * GC * 2, "the T staging tile reuses the A area");
    __shared__ __align__(16) float sA[tri_off(GC)];  // A packed columns; then T diag(beta), bf16 [64][64]
    __shared__ __align__(16) float sD[GC * 16];      // diagonal blocks of T, row-major per block
    __shared__ float sG[2][GC], sB[GC];
    // wavefront-local order of LDS traffic: later LDS reads see the lanes' earlier writes
    auto wave_sync = [] __attribute__((always_inline)) () { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };

    // blockIdx -> unit u = slot * H + h, in runs of kPrepXcdRun units per XCD (workgroups go
    // round-robin over the 8 XCDs)
    const int xcd = blockIdx.x & 7, idx = blockIdx.x >> 3;
    const int u = (idx / kPrepXcdRun) * (8 * kPrepXcdRun) + xcd * kPrepXcdRun + idx % kPrepXcdRun;
    if (u >= H * n_slots) return;
    const int slot = u / H, h = u % H;
    const int hk = h / (H / HK);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    int b, t0, L, ci;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L, ci)) return;

    // gates of the chunk (both wavefronts; padded tokens get g = 0)
    const size_t gi = (size_t)(b * T + t0 + min(lane, L - 1)) * H + h;
    const float G = wave_inclusive_scan(lane < L ? load_gate(g, gs, gi, h) : 0.f);
    float* sGw = sG[wave];
    sGw[lane] = G;
    uint8_t* rec = fac + ((size_t)slot * H + h) * gdn_factor_bytes(2);
    bf16_t* gT = reinterpret_cast<bf16_t*>(rec);
    bf16_t* gP = gT + GC * GC;
    float* gC = reinterpret_cast<float*>(gP + GC * GC);
    // K rows of the chunk. Rows past a partial chunk's end repeat its last token: they only reach
    // entries that are never read or are cancelled exactly (rows of A scaled by beta = 0; columns of
    // P and W that meet padded tokens only, whose e and T diag(beta) columns are zero)
    bf16x8 kf[4][KP];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
        const int t = 16 * R + ln;
        const bf16_t* row = k + ((size_t)(b * T + t0 + min(t, L - 1)) * HK + hk) * KD + 8 * lg;
#pragma unroll
        for (int p = 0; p < KP; ++p) kf[R][p] = *reinterpret_cast<const bf16x8*>(row + 32 * p);
    }

    // W = K_c K_{c-1}^T, as the A operand of W (e R)_{c-1} (a sequence's first chunk has no
    // predecessor: its W is formed from its own first row and never read): fragment (u, p) holds, for lane (ln, lg), W[16 u + ln][32 p + 4 lg + j]
    // then W[16 u + ln][32 p + 16 + 4 lg + j]. The C tile of K_{c-1} K_c^T (rows s, columns t) is
    // exactly that lane content, so each fragment pairs two of those tiles without any shuffle.
    // Wavefront pp forms the fragments (u, pp) from the row tiles 2 pp, 2 pp + 1 of the preceding
    // (always full) chunk of the same sequence.
    auto make_w = [&](int pp) __attribute__((always_inline)) {
        bf16_t* gW = reinterpret_cast<bf16_t*>(rec + kGdnWOffset);
        bf16x8 kq[2][KP];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int t = 16 * (2 * pp + s2) + ln;
            const int pt = ci > 0 ? t0 - GC + t : t0;
            const bf16_t* row = k + ((size_t)(b * T + pt) * HK + hk) * KD + 8 * lg;
#pragma unroll
            for (int p = 0; p < KP; ++p) kq[s2][p] = *reinterpret_cast<const bf16x8*>(row + 32 * p);
        }
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
            f32x4 w0 = zero4(), w1 = zero4();
#pragma unroll
            for (int p = 0; p < KP; ++p) {
                w0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq[0][p], kf[uu][p], w0, 0, 0, 0);
                w1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kq[1][p], kf[uu][p], w1, 0, 0, 0);
            }
            const i16x4 lo = Elem<bf16_t>::pack(w0), hi = Elem<bf16_t>::pack(w1);
            *reinterpret_cast<i16x8*>(gW + ((2 * uu + pp) * 64 + lane) * 8) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
    };

    auto role0 = [&]() __attribute__((always_inline)) {
        const float bv = lane < L ? beta[gi] : 0.f;
        sB[lane] = bv;
        {
            const float GL = __shfl(G, 63, 64);
            gC[lane] = expf(G);
            gC[64 + lane] = expf(GL - G);
            gC[128 + lane] = bv;
            gC[192 + lane] = G;
        }
        wave_sync();
        // A on the 10 lower tiles: C tile lane (ln, lg) holds (K K^T)[16 ti + 4 lg + r][16 tj + ln]
#pragma unroll
        for (int tt = 0; tt < 10; ++tt) {
            const int ti = (tt >= 1) + (tt >= 3) + (tt >= 6);
            const int tj = tt - ti * (ti + 1) / 2;
            f32x4 a = zero4();
#pragma unroll
            for (int p = 0; p < KP; ++p) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ti][p], kf[tj][p], a, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 16 * ti + 4 * lg + r, i = 16 * tj + ln;
                const float d = __expf(fminf(sGw[t] - sGw[i], 0.f));
                if (i < t) sA[col_off(i) + (t - i - 1)] = sB[t] * d * a[r];
            }
        }
        if (want_w) make_w(0);
        wave_sync();
        // T = (I + A)^-1 by 16x16 blocks (A strictly lower, float32). The diagonal blocks
        // D_b = (I + A_bb)^-1 come from forward substitution, lane (b, jj) holding column jj of D_b
        // (15 steps for all four blocks at once); the others from block row i of (I + A) T = I,
        //   T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj  (T_jj = D_j),
        // one block diagonal i - j at a time, as float32 MFMA block products (sf_device.h).
        const int db = lane >> 4, dj = lane & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == dj) ? 1.f : 0.f;
#pragma unroll
        for (int t = 0; t < 15; ++t) {
            const float* col = sA + col_off(16 * db + t);  // rows 16 db + t + 1 .. of column 16 db + t
            const float xt = x[t];
#pragma unroll
            for (int r = t + 1; r < 16; ++r) x[r] -= col[r - t - 1] * xt;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sD[(16 * db + r) * 16 + dj] = x[r];
        wave_sync();
        // fragments: A operand lane (ln, lg) <- M[ln][4 lg + q], B operand <- M[4 lg + q][ln]
        auto d_a = [&](int i) __attribute__((always_inline)) { return *reinterpret_cast<const f32x4*>(sD + (16 * i + ln) * 16 + 4 * lg); };
        auto d_b = [&](int j) __attribute__((always_inline)) {
            f32x4 r;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) r[qq] = sD[(16 * j + 4 * lg + qq) * 16 + ln];
            return r;
        };
        auto a_a = [&](int i, int j) __attribute__((always_inline)) {  // block A_ij, i > j
            f32x4 r;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int c = 16 * j + 4 * lg + qq;
                r[qq] = sA[col_off(c) + (16 * i + ln) - c - 1];
            }
            return r;
        };
        f32x4 Tb[4][4];  // Tb[i][j], i > j, C tile: lane (ln, lg) holds T[16 i + 4 lg + r][16 j + ln]
#pragma unroll
        for (int dd = 1; dd < 4; ++dd)
#pragma unroll
            for (int j = 0; j + dd < 4; ++j) {
                const int i = j + dd;
                f32x4 uu = Elem<float>::mma(zero4(), a_a(i, j), d_b(j));
#pragma unroll
                for (int kk = j + 1; kk < i; ++kk) uu = Elem<float>::mma(uu, a_a(i, kk), Tb[kk][j]);
                Tb[i][j] = Elem<float>::mma(zero4(), d_a(i), uu) * -1.f;
            }
        wave_sync();
        // T diag(beta) (column j scaled by beta_j, zero past the chunk's end) into the staging tile
        // over the A area; the two blocks right of the diagonal that the fragments cover are zero
        bf16_t* sS = reinterpret_cast<bf16_t*>(sA);
#pragma unroll
        for (int r = 0; r < 16; ++r) sS[(16 * db + r) * GC + 16 * db + dj] = f2bf(x[r] * bv);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float bj = sB[16 * j + ln];
#pragma unroll
            for (int i = j + 1; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[(16 * i + 4 * lg + r) * GC + 16 * j + ln] = f2bf(Tb[i][j][r] * bj);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sS[(4 * lg + r) * GC + 16 + ln] = 0;
            sS[(32 + 4 * lg + r) * GC + 48 + ln] = 0;
        }
        wave_sync();
        store_tri_frags(sS, GC, gT);
    };
    auto role1 = [&]() __attribute__((always_inline)) {
        wave_sync();
        if constexpr (WANT_P) {
            // P^T tiles, K rows (A operand, rows s) against Q rows (B operand, columns t): C tile lane
            // (ln, lg) holds P[16 ti + ln][16 tj + 4 lg + r], which is fragment (ti, tj / 2)'s lane
            // content (first or second half)
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const int t = 16 * ti + ln;
                bf16x8 qf[KP];
                const bf16_t* row = q + ((size_t)(b * T + t0 + min(t, L - 1)) * HK + hk) * KD + 8 * lg;
#pragma unroll
                for (int p = 0; p < KP; ++p) qf[p] = *reinterpret_cast<const bf16x8*>(row + 32 * p);
                const float Gt = sGw[t];
                f32x4 PT[4];
#pragma unroll
                for (int tj = 0; tj < 4; ++tj) {
                    PT[tj] = zero4();
                    if (tj <= ti) {
#pragma unroll
                        for (int p = 0; p < KP; ++p) PT[tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tj][p], qf[p], PT[tj], 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int i = 16 * tj + 4 * lg + r;
                            const float d = __expf(fminf(Gt - sGw[i], 0.f));
                            PT[tj][r] = i <= t ? scale * d * PT[tj][r] : 0.f;
                        }
                    }
                }
#pragma unroll
                for (int p = 0; p <= ti / 2; ++p) {
                    const i16x4 lo = Elem<bf16_t>::pack(PT[2 * p]), hi = Elem<bf16_t>::pack(PT[2 * p + 1]);
                    *reinterpret_cast<i16x8*>(gP + (tri_frag(ti, p) * 64 + lane) * 8) = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
            }
        }
        if (want_w) make_w(1);
    };
    if constexpr (NW == 2) {
        if (wave == 0)
            role0();
        else
            role1();
    } else {
        role0();
        role1();
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
// ST + Out, bf16: one workgroup = one 16-row state slice of one chain, eight
// wavefronts.
//
//  With S_c the entry state of chunk c, the key-state product is split as
//        X_c = K_c S_c^T = Gamma_L(c-1) Z_c + W_c (e R)_{c-1},
//        Z_c = K_c S_{c-1}^T,   W_c = K_c K_{c-1}^T  (from the Pre stage),
//  so one chunk step is two independent streams, each on its own SIMD:
//  - wavefront 0, residual:  X_c -> Y_c = V_c - diag(Gamma) X_c
//                            -> R_c = T_c diag(beta) Y_c -> (e R)_c
//  - wavefronts 1 and 2, state, one half of the key columns each:
//                            S_c = Gamma_L S_{c-1} + K_{c-1}^T (e R)_{c-1}
//                            -> Z_{c+1} = K_{c+1} S_c^T (each its half of the sum over k),
//    the slice state held in float32 MFMA accumulators for the whole chain.
//  Each step needs only (e R)_{c-1} and Z_c from the previous one; the
//  wavefronts swap them through LDS once per chunk. Within a wavefront the
//  C tile of each product is the operand of the next as it stands
//  (sf_device.h).
//  - Wavefronts 3 and 7 form the output, two token tiles each: in step c they
//    read their Q_c and P_c fragments (P from the Pre stage) from LDS into
//    registers; in step c+1 they form
//    O_c^T = scale diag(Gamma) (S_c Q_c^T) + R_c^T P_c^T from the bf16 state
//    and residual fragments the chain leaves in LDS, and store it (8-byte row
//    pieces) at the start of step c+2: stores issued mid-step, while the
//    feeders' loads are in flight, stretch the step more.
//  - Wavefronts 4, 5 and 6 feed everyone with 16-byte direct loads into LDS
//    (no register staging; one wavefront alone issues them too slowly): in
//    step c they move K of chunk c+2, Q, T, W, V and coefficients of chunk
//    c+1. K and Q rows go four whole rows per load.
//  One workgroup barrier per chunk.
//
// State tiles: S[kt], kt = 2p + h, is the C tile of S^T whose row 4 lg + j
// stands for key column k = 32 p + 8 lg + 4 h + j and whose column ln for
// state row row0 + ln. The pairs (S[2p], S[2p+1]) then give lane group lg the
// eight consecutive columns 32 p + 8 lg .. + 7, so K and Q rows enter the
// products as plain 16-byte row fragments.
//
// K and Q in LDS: RowBlock layout (sf_device.h).
// ---------------------------------------------------------------------------

template <int KD, bool SUMMARY>
struct ChainLds {
    typedef RowBlock<KD> RBk;
    static constexpr int KP = KD / 32, KB = KD / 16;
    // K of chunk c: row fragments in step c-1 (Z_c), transposed in step c (for the update with
    // (e R)_c); loaded in step c-2
    static constexpr int NK = 3;
    static constexpr int KBUF = RBk::BYTES;
    // Q of chunk c: read in step c (the Q fragments kept for O_c); loaded in step c-1
    static constexpr int NQ = 2;
    // T, W, V, coefficients and P of chunk c: step c; loaded in step c-1
    static constexpr int NT = 2;
    static constexpr int OFF_T = 0;                                  // kTriFrags fragments of 1 KB
    static constexpr int OFF_W = OFF_T + kTriFrags * 1024;           // 8 fragments of 1 KB
    static constexpr int OFF_V = OFF_W + 8 * 1024;                   // V slice [64][16] bf16
    static constexpr int OFF_C = OFF_V + GC * 16 * 2;                // coefficients float[256]
    static constexpr int OFF_P = OFF_C + 256 * 4;                    // kTriFrags fragments of 1 KB
    static constexpr int TBUF = OFF_P + (SUMMARY ? 0 : kTriFrags * 1024);
    static constexpr int OFF_KR = 0;
    static constexpr int OFF_QR = OFF_KR + NK * KBUF;
    static constexpr int OFF_TR = OFF_QR + (SUMMARY ? 0 : NQ * KBUF);
    static constexpr int OFF_Z = OFF_TR + NT * TBUF;                 // [2 halves][2][4][64] x 16 B  float Z
    static constexpr int ZHALF = 2 * 4 * 1024;
    static constexpr int OFF_ER = OFF_Z + 2 * ZHALF;                 // [2][4][64] x 8 B   bf16 e R
    static constexpr int OFF_SF = OFF_ER + 2 * 4 * 512;              // [2][KB][64] x 8 B  bf16 state
    static constexpr int OFF_RB = OFF_SF + (SUMMARY ? 0 : 2 * KB * 512);  // [2][4][64] x 8 B  bf16 R
    static constexpr int OFF_JUNK = OFF_RB + (SUMMARY ? 0 : 2 * 4 * 512);  // 256 B sink of cache warm-up loads
    static constexpr int BYTES = OFF_JUNK + 256;
    static_assert(BYTES <= 160 * 1024, "chain LDS plan exceeds the CU's 160 KB");
};

// s_waitcnt immediate for lgkmcnt(0) with the vector-memory and export counts left alone (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitLgkm0 = 0xC07F;


template <int KD, bool SUMMARY>
__global__ __launch_bounds__(512) void gdn_chain_1w_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const uint8_t* __restrict__ fac, int T, int H, int HK, int V, int n_seq, int nc, int nvb,
    float scale, bf16_t* __restrict__ out, float* __restrict__ ht, float* __restrict__ Mout) {
    typedef ChainLds<KD, SUMMARY> SM;
    typedef RowBlock<KD> RBk;
    typedef Elem<bf16_t> El;
    constexpr int KP = SM::KP, KB = SM::KB;
    constexpr int UST = (16 / RBk::RPB) * 1024;  // byte step of one 16-row token tile in a row block

    __shared__ __align__(16) uint8_t smem[SM::BYTES];
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    lds_u8* const lds0 = (lds_u8*)smem;
    auto opaque = [](lds_u8* p) __attribute__((always_inline)) { asm volatile("" : "+v"(p)); return p; };

    int chain, vb;
    xcd_split(blockIdx.x, nvb, chain, vb);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, hk = h / (H / HK);
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    // Role numbers below: the CU places wavefront w of a workgroup on SIMD w % 4, so the two output
    // roles (3 and 7), the heaviest in issued instructions, run as wavefronts 3 and 5, each beside a
    // light role on its SIMD (role 5 runs as wavefront 7).
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wid == 5 ? 7 : wid == 7 ? 5 : wid;
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
    auto kbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_KR + (c % SM::NK) * SM::KBUF; };
    auto qbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_QR + (c % SM::NQ) * SM::KBUF; };
    auto tbuf = [&](int c) __attribute__((always_inline)) { return lds0 + SM::OFF_TR + (c % SM::NT) * SM::TBUF; };
    auto record = [&](int c) __attribute__((always_inline)) {
        return fac + ((size_t)(slot0 + c) * H + h) * rec_bytes;
    };
    // lane offsets of row fragment (0, p) (16 rows, one 16-byte piece) and of the transposed-read
    // pointer for column pair p (token 4 lg + ln/4, piece 4 p + ln%4) in a row block
    auto roff_row = [&](int p) __attribute__((always_inline)) { return RBk::off(ln, 4 * p + lg); };
    auto roff_tr = [&](int p) __attribute__((always_inline)) { return RBk::off(4 * lg + (ln >> 2), 4 * p + (ln & 3)); };
    // Each role below runs its own loop with two barriers before the first chunk and one per
    // chunk, so the roles' registers never overlap; every wavefront's own memory traffic is
    // complete (explicit waits) before it reaches a barrier.
    auto barrier = [] __attribute__((always_inline)) () { asm volatile("s_barrier" ::: "memory"); };

    if (wave == 0) {
        // ================= residual stream =================
        const int off_frag = lane * 16;                                             // W, T fragments
        const int off_coef = 16 * lg;                                               // coefficient rows
        const int off_v = ((4 * lg + (ln >> 2)) * 16 + 4 * (ln & 3)) * 2;           // V read transposed
        const uint32_t vmask = vrows ? 0xffffffffu : 0u;  // transition rows (summary) carry no values
        barrier();
        barrier();
        float glp = 1.f;    // Gamma_L of chunk c-1
        i16x4 ERp[4];       // (e R)_{c-1}
        for (int c = 0; c < nch; ++c) {
            lds_u8* tb = tbuf(c);
            lds_u8* xb = lds0 + SM::OFF_Z + (c & 1) * 4 * 1024 + off_frag;            // Z halves, 16 B / lane
            lds_u8* eb = lds0 + SM::OFF_ER + (c & 1) * 4 * 512 + lane * 8;            // e R, R fragments
            lds_u8* fb = tb + off_frag;
            lds_u8* cb = tb + SM::OFF_C + off_coef;
            lds_u8* vb_ = tb + SM::OFF_V + off_v;
            asm volatile("" : "+v"(xb), "+v"(eb), "+v"(fb), "+v"(cb), "+v"(vb_));
            f32x4 X[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) X[u] = *(const lds_f32x4*)(xb + u * 1024) + *(const lds_f32x4*)(xb + SM::ZHALF + u * 1024);
            bf16x8 Wf[8], Tf[kTriFrags];
            f32x4 gam[4], ec[4];
            i16x4 Vf[4];
#pragma unroll
            for (int f = 0; f < 8; ++f) Wf[f] = *(const lds_bf16x8*)(fb + SM::OFF_W + f * 1024);
#pragma unroll
            for (int f = 0; f < kTriFrags; ++f) Tf[f] = *(const lds_bf16x8*)(fb + SM::OFF_T + f * 1024);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                gam[u] = *(const lds_f32x4*)(cb + 64 * u);
                ec[u] = *(const lds_f32x4*)(cb + 256 + 64 * u);
                const i16x4 vx = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb_ + 16 * u * 16 * 2));
                typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                Vf[u] = __builtin_bit_cast(i16x4, __builtin_bit_cast(u32x2, vx) & vmask);
            }
            const float gl = *(const __attribute__((address_space(3))) float*)(tb + SM::OFF_C + 63 * 4);
            // X_c = Gamma_L(c-1) Z_c + W_c (e R)_{c-1}
            if (c > 0) {
                const bf16x8 E01 = cat8(ERp[0], ERp[1]), E23 = cat8(ERp[2], ERp[3]);
#pragma unroll
                for (int u = 0; u < 4; ++u) X[u] = mma32(Wf[2 * u + 1], E23, mma32(Wf[2 * u], E01, X[u] * glp));
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
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                ERp[ti] = El::pack(R[ti] * ec[ti]);
                *(lds_i16x4*)(eb + ti * 512) = ERp[ti];
            }
            if constexpr (!SUMMARY) {
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) *(lds_i16x4*)(eb + (SM::OFF_RB - SM::OFF_ER) + ti * 512) = El::pack(R[ti]);
            }
            glp = gl;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            barrier();
        }
    } else if (wave == 1 || wave == 2) {
        // ================= state stream, one half of the key columns per wavefront =================
        // wavefront 1 holds key tiles [0, KB/2), wavefront 2 [KB/2, KB): each updates its half of the
        // state and forms its half of the sum over k in Z; the residual stream adds the two halves
        constexpr int KH = KB / 2, KPH = KP / 2;
        const int half = wave - 1, kt0 = half * KH, p0 = half * KPH;
        f32x4 S[KH];
#pragma unroll
        for (int i = 0; i < KH; ++i) {
            const int kt = kt0 + i;
            const int kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1), row = row0 + ln;
            if constexpr (!SUMMARY) {
                S[i] = h0 ? *reinterpret_cast<const f32x4*>(h0 + (((size_t)n * H + h) * V + row) * KD + kk) : zero4();
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[i][r] = (!vrows && kk + r == row - V) ? 1.f : 0.f;
            }
        }
        int orow[KPH], otr[KPH];
#pragma unroll
        for (int i = 0; i < KPH; ++i) {
            orow[i] = roff_row(p0 + i);
            otr[i] = roff_tr(p0 + i);
        }
        bf16x8 Kf[4][KPH];
        auto read_krow = [&](int c) __attribute__((always_inline)) {  // K_c rows, own column pairs
#pragma unroll
            for (int i = 0; i < KPH; ++i) {
                lds_u8* B = opaque(kbuf(c) + orow[i]);
#pragma unroll
                for (int u = 0; u < 4; ++u) Kf[u][i] = *(lds_bf16x8*)(B + u * UST);
            }
        };
        // K^T fragments of chunk c, own key tiles: transposed reads of the row blocks; lane i of
        // group g points at token 16 u + 4 g + i/4, columns 32 p + 8 (i%4) + 4 h
        i16x4 Ka[KH][4];
        auto read_kt = [&](int c) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < KPH; ++i) {
                lds_u8* B = opaque(kbuf(c) + otr[i]);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        Ka[2 * i + hh][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(B + u * UST + 8 * hh));
            }
        };
        i16x4 ER[4];
        auto read_er = [&](int c) __attribute__((always_inline)) {  // (e R)_c from the residual stream
            lds_u8* B = opaque(lds0 + SM::OFF_ER + (c & 1) * 4 * 512 + lane * 8);
#pragma unroll
            for (int ti = 0; ti < 4; ++ti) ER[ti] = *(lds_i16x4*)(B + ti * 512);
        };
        auto update = [&](float glp) __attribute__((always_inline)) {  // S <- glp S + K^T (e R)
            const bf16x8 E01 = cat8(ER[0], ER[1]), E23 = cat8(ER[2], ER[3]);
#pragma unroll
            for (int i = 0; i < KH; ++i) {
                f32x4 acc = S[i] * glp;
                acc = mma32(cat8(Ka[i][0], Ka[i][1]), E01, acc);
                acc = mma32(cat8(Ka[i][2], Ka[i][3]), E23, acc);
                S[i] = acc;
            }
        };
        auto pack_state = [&](int c, i16x4 (&Sf)[KH]) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < KH; ++i) Sf[i] = El::pack(S[i]);
            if constexpr (!SUMMARY) {
                lds_u8* B = opaque(lds0 + SM::OFF_SF + (c & 1) * KB * 512 + kt0 * 512 + lane * 8);
#pragma unroll
                for (int i = 0; i < KH; ++i) *(lds_i16x4*)(B + i * 512) = Sf[i];
            }
        };
        // partial Z_c = K_c[:, own columns] S[:, own columns]^T, left for the residual stream
        auto z_of = [&](const i16x4 (&Sf)[KH], f32x4 (&Zn)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                Zn[u] = zero4();
#pragma unroll
                for (int i = 0; i < KPH; ++i) Zn[u] = mma32(Kf[u][i], cat8(Sf[2 * i], Sf[2 * i + 1]), Zn[u]);
            }
        };
        auto store_z = [&](int c, const f32x4 (&Zn)[4]) __attribute__((always_inline)) {
            lds_u8* zb = opaque(lds0 + SM::OFF_Z + half * SM::ZHALF + (c & 1) * 4 * 1024 + lane * 16);
#pragma unroll
            for (int u = 0; u < 4; ++u) *(lds_f32x4*)(zb + u * 1024) = Zn[u];
        };
        barrier();
        if (nch > 0) {
            read_krow(0);
            i16x4 Sf[KH];
#pragma unroll
            for (int i = 0; i < KH; ++i) Sf[i] = El::pack(S[i]);
            f32x4 Zn[4];
            z_of(Sf, Zn);
            store_z(0, Zn);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        barrier();
        float glp = 1.f;
        // The LDS wait counter holds at most 15 operations in flight and counts them in issue order,
        // so the phases below are pinned (sched_barrier) such that each wait is on the newest group:
        // e R -> (K_{c+1} rows out) -> update -> bf16 state out -> Z (waits on K rows only)
        // -> (K_c^T out) -> Z out.
        for (int c = 0; c < nch; ++c) {
            const bool more = c + 1 < nch;
            const float gl = *(const __attribute__((address_space(3))) float*)(tbuf(c) + SM::OFF_C + 63 * 4);
            if (c > 0) read_er(c - 1);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // (the compiler's counter model sees this form)
            __builtin_amdgcn_sched_barrier(0);
            if (more) read_krow(c + 1);
            __builtin_amdgcn_sched_barrier(0);
            // S_c = Gamma_L(c-1) S_{c-1} + K_{c-1}^T (e R)_{c-1}
            if (c > 0) update(glp);
            i16x4 Sf[KH];
            pack_state(c, Sf);
            __builtin_amdgcn_sched_barrier(0);
            if (more) {
                // Z_{c+1} = K_{c+1} S_c^T (own half of the sum)
                f32x4 Zn[4];
                z_of(Sf, Zn);
                __builtin_amdgcn_sched_barrier(0);
                // K^T of chunk c for the next update: lands while Z finishes and the barrier is waited on
                read_kt(c);
                store_z(c + 1, Zn);
            } else {
                read_kt(c);
            }
            glp = gl;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            barrier();
        }
        // exit state S_nch = Gamma_L S_{nch-1} + K_{nch-1}^T (e R)_{nch-1}
        if (nch > 0) {
            read_er(nch - 1);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            update(glp);
        }
#pragma unroll
        for (int i = 0; i < KH; ++i) {
            const int kt = kt0 + i;
            const int kk = 32 * (kt >> 1) + 8 * lg + 4 * (kt & 1), row = row0 + ln;
            if (vrows) {
                if (ht) *reinterpret_cast<f32x4*>(ht + (((size_t)n * H + h) * V + row) * KD + kk) = S[i];
            } else if constexpr (SUMMARY) {
                *reinterpret_cast<f32x4*>(Mout + (((size_t)n * H + h) * KD + (row - V)) * KD + kk) = S[i];
            }
        }
    } else if (wave >= 4 && wave <= 6) {
        // ================= feeders: direct loads into LDS, three wavefronts =================
        // One wavefront issues these loads at a fraction of the rate several do, so the chunk's loads
        // are split by kind: wavefront 4 the K rows (and a cache warm-up), 5 the Q rows and the P part
        // of the record, 6 the other record parts (T, W, coefficients) and the V slice. Every lane offset is computed once; a load is
        // then a scalar base, an LDS destination and the load itself. Rows past the end of a partial
        // chunk repeat its last token (finite values that the stored T diag(beta), W and e = 0 keep out
        // of every result, and that the output never stores).
        const int fi = wave - 4;
        constexpr int NPAT = 16 / RBk::RPB;  // the swizzle repeats every 16 rows = NPAT row blocks
        const size_t krs = (size_t)HK * KD * 2, vrs = (size_t)H * V * 2;  // token strides (bytes)
        // row-block loads: instruction m, lane l -> row m RPB + l / PCS, piece (l % PCS) ^ swz(row)
        uint32_t rowoff[NPAT];
#pragma unroll
        for (int j = 0; j < NPAT; ++j) {
            const int r = j * RBk::RPB + lane / RBk::PCS;
            rowoff[j] = (uint32_t)((lane / RBk::PCS) * krs) + 16u * (uint32_t)((lane % RBk::PCS) ^ RBk::swz(r));
        }
        auto feed_rows = [&](const bf16_t* src, int c, lds_u8* dst) __attribute__((always_inline)) {
            const int t0 = bos + c * GC, L = min(GC, eos - t0);
            const uint8_t* base = reinterpret_cast<const uint8_t*>(src + ((size_t)(b * T + t0) * HK + hk) * KD);
            if (L == GC) {
#pragma unroll
                for (int m = 0; m < RBk::NLOAD; ++m)
                    load_lds16(base + (size_t)(m * RBk::RPB) * krs + rowoff[m % NPAT], (uint8_t*)(dst + m * 1024));
            } else {
#pragma unroll
                for (int m = 0; m < RBk::NLOAD; ++m) {
                    const int r = m * RBk::RPB + lane / RBk::PCS, pc = lane % RBk::PCS;
                    const int t = min(r, L - 1);
                    load_lds16(base + (size_t)t * krs + 16 * (pc ^ RBk::swz(r)), (uint8_t*)(dst + m * 1024));
                }
            }
        };
        const uint32_t voff = (uint32_t)((lane >> 1) * vrs) + (uint32_t)(((vrows ? row0 : 0) + 8 * (lane & 1)) * 2);
        auto feed_t = [&](int c) __attribute__((always_inline)) {
            const int t0 = bos + c * GC, L = min(GC, eos - t0);
            lds_u8* B = tbuf(c);
            const uint8_t* rec = record(c) + lane * 16;
#pragma unroll
            for (int f = 0; f < kTriFrags; ++f) load_lds16(rec + f * 1024, (uint8_t*)(B + SM::OFF_T + f * 1024));
#pragma unroll
            for (int f = 0; f < 8; ++f) load_lds16(rec + kGdnWOffset + f * 1024, (uint8_t*)(B + SM::OFF_W + f * 1024));
            load_lds16(rec + 2 * GC * GC * 2, (uint8_t*)(B + SM::OFF_C));
            // V slice [64][16]; transition-row slices (summary mode) never read it: they load value rows 0..15
            const uint8_t* vb0 = reinterpret_cast<const uint8_t*>(v + (size_t)(b * T + t0) * H * V + (size_t)h * V);
#pragma unroll
            for (int hv = 0; hv < 2; ++hv) {
                if (L == GC) {
                    load_lds16(vb0 + (size_t)(32 * hv) * vrs + voff, (uint8_t*)(B + SM::OFF_V + hv * 1024));
                } else {
                    const int t = min(32 * hv + (lane >> 1), L - 1);
                    load_lds16(vb0 + (size_t)t * vrs + ((vrows ? row0 : 0) + 8 * (lane & 1)) * 2,
                               (uint8_t*)(B + SM::OFF_V + hv * 1024));
                }
            }
        };
        auto feed_p = [&](int c) __attribute__((always_inline)) {
            const uint8_t* rec = record(c) + GC * GC * 2 + lane * 16;
#pragma unroll
            for (int f = 0; f < kTriFrags; ++f) load_lds16(rec + f * 1024, (uint8_t*)(tbuf(c) + SM::OFF_P + f * 1024));
        };
        // Cache warm-up (wavefront 4): the direct loads run one step ahead, and the lines of chunk c+3 are
        // touched now (one 4-byte load per 128-byte line: the rows of K, Q and V of the head, the T, W,
        // coefficient and P parts of the record) and sit in this XCD's L2 when their loads come. The
        // head's slices share the lines: slice vb touches line li = (64 vb + lane) mod (list length) and,
        // with P, line min(li + 512, last) of the chunk's list (duplicates are harmless).
        constexpr int NLINES = 504 + (SUMMARY ? 0 : 48);
        constexpr int NWARM = NLINES > 512 ? 2 : 1;
        auto warm_line = [&](int c, int li) __attribute__((always_inline)) {
            const int t0 = bos + c * GC, L = min(GC, eos - t0);
            const uint8_t* a;
            if (li < 256) {        // K rows (0..127), Q rows (128..255): two 128-byte lines per row
                const int t = min((li & 127) >> 1, L - 1);
                const bf16_t* base = li < 128 ? k : (SUMMARY ? k : q);
                a = reinterpret_cast<const uint8_t*>(base + ((size_t)(b * T + t0 + t) * HK + hk) * KD) + (li & 1) * (KD >= 128 ? 128 : 0);
            } else if (li < 384) { // V rows of the head (two lines per token)
                const int t = min((li - 256) >> 1, L - 1);
                a = reinterpret_cast<const uint8_t*>(v + ((size_t)(b * T + t0 + t) * H + h) * V) + (li & 1) * (V >= 128 ? 128 : 0);
            } else {               // record: T (48 lines), coefficients (8), W (64), P (48)
                const int r = li - 384;
                const size_t off = r < 48    ? (size_t)r * 128
                                   : r < 56  ? (size_t)2 * GC * GC * 2 + (r - 48) * 128
                                   : r < 120 ? kGdnWOffset + (size_t)(r - 56) * 128
                                             : (size_t)GC * GC * 2 + (r - 120) * 128;
                a = record(c) + off;
            }
            __builtin_amdgcn_global_load_lds(a, (__attribute__((address_space(3))) void*)(smem + SM::OFF_JUNK), 4, 0, 0);
        };
        const int li = (64 * vb + lane) % NLINES;
        auto warm = [&](int c) __attribute__((always_inline)) {
            warm_line(c, li);
            if constexpr (NWARM == 2) warm_line(c, min(li + 512, NLINES - 1));
        };
        // one step of this wavefront's share: chunk c+2 of K, chunk c+1 of Q and of the record/V
        auto feed = [&](int cK, int cR) __attribute__((always_inline)) {
            if (fi == 0) {
                if (cK < nch) feed_rows(k, cK, kbuf(cK));
            } else if (fi == 1) {
                if constexpr (!SUMMARY)
                    if (cR < nch) {
                        feed_rows(q, cR, qbuf(cR));
                        feed_p(cR);
                    }
            } else {
                if (cR < nch) feed_t(cR);
            }
        };
        // everything read before the first chunk step and in it has landed before the first barrier
        if (fi == 0) {
            if (nch > 2) warm(2);
            if (nch > 1) feed_rows(k, 1, kbuf(1));
        }
        feed(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier();
        barrier();
        for (int c = 0; c < nch; ++c) {
            feed(c + 2, c + 1);
            if (fi == 0 && c + 3 < nch) {
                // issued after this step's loads: the wait below leaves only the warm-up in flight
                // (loads complete in issue order); touching chunk c+4 instead measured 5 us slower
                warm(c + 3);
                if constexpr (NWARM == 2)
                    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
                else
                    asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            barrier();
        }
    } else {
        // ================= output: wavefront 3 tiles {0, 3}, wavefront 7 tiles {1, 2} =================
        barrier();
        barrier();
        if constexpr (!SUMMARY) {
            struct OutRegs {
                bf16x8 Qf[2][KP], Pf[2][2];
                float gq[2];
            };
            auto tile_of = [&](int i) __attribute__((always_inline)) { return wave == 3 ? 3 * i : 1 + i; };
            int orow[KP];
#pragma unroll
            for (int p = 0; p < KP; ++p) orow[p] = roff_row(p);
            // chunk c's Q fragments and P fragments of own tiles, from LDS. The stored P fragment (tt, p)
            // is, per lane, P[16 tt + ln][32 p + 4 lg + j] then P[16 tt + ln][32 p + 16 + 4 lg + j]: the
            // B operand of the product with the R fragment pair p of the same tokens.
            auto build = [&](int c, OutRegs& F) __attribute__((always_inline)) {
                lds_u8* cb = tbuf(c) + SM::OFF_C;
                lds_u8* pb = opaque(tbuf(c) + SM::OFF_P + lane * 16);
                lds_u8* qb[KP];
#pragma unroll
                for (int p = 0; p < KP; ++p) qb[p] = opaque(qbuf(c) + orow[p]);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int tt = tile_of(i);
#pragma unroll
                    for (int p = 0; p < KP; ++p) F.Qf[i][p] = *(lds_bf16x8*)(qb[p] + tt * UST);
                    F.gq[i] = *(const __attribute__((address_space(3))) float*)(cb + (16 * tt + ln) * 4);
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        if (p <= tt / 2) F.Pf[i][p] = *(lds_bf16x8*)(pb + tri_frag(tt, p) * 1024);
                }
            };
            // O pieces formed in one step and stored at the start of the next
            i16x4 pend_o[2];
            bf16_t* pend_at[2];
            bool pend[2] = {false, false};
            auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    if (pend[i]) *reinterpret_cast<i16x4*>(pend_at[i]) = pend_o[i];
            };
            // O of chunk c: stored now (last chunk) or left pending
            auto emit = [&](int c, const OutRegs& E, bool now) __attribute__((always_inline)) {
                const int t0 = bos + c * GC, L = min(GC, eos - t0);
                lds_u8* sb = opaque(lds0 + SM::OFF_SF + (c & 1) * KB * 512 + lane * 8);
                lds_u8* rb = opaque(lds0 + SM::OFF_RB + (c & 1) * 4 * 512 + lane * 8);
                i16x4 Sf[KB], Rb[4];
#pragma unroll
                for (int kt = 0; kt < KB; ++kt) Sf[kt] = *(lds_i16x4*)(sb + kt * 512);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) Rb[ti] = *(lds_i16x4*)(rb + ti * 512);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int tt = tile_of(i);
                    f32x4 qs = zero4();
#pragma unroll
                    for (int p = 0; p < KP; ++p) qs = mma32(cat8(Sf[2 * p], Sf[2 * p + 1]), E.Qf[i][p], qs);
                    f32x4 o = qs * (E.gq[i] * scale);
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        if (p <= tt / 2) o = mma32(cat8(Rb[2 * p], Rb[2 * p + 1]), E.Pf[i][p], o);
                    const int t = 16 * tt + ln;
                    bf16_t* at = out + ((size_t)(b * T + t0 + t) * H + h) * V + row0 + 4 * lg;
                    if (now) {
                        if (t < L) *reinterpret_cast<i16x4*>(at) = El::pack(o);
                    } else {
                        pend_o[i] = El::pack(o);
                        pend_at[i] = at;
                        pend[i] = t < L;
                    }
                }
            };
            // step c: store chunk c-2, read chunk c's operands into F (Q_c, P_c resident now),
            // form chunk c-1 from E
            auto step = [&](int c, OutRegs& F, const OutRegs& E) __attribute__((always_inline)) {
                flush();
                build(c, F);
                if (c > 0) emit(c - 1, E, false);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                barrier();
            };
            OutRegs RA, RB;
            for (int c = 0; c < nch; c += 2) {
                step(c, RA, RB);
                if (c + 1 < nch) step(c + 1, RB, RA);
            }
            flush();
            if (nch > 0) emit(nch - 1, (nch - 1) & 1 ? RB : RA, true);
        } else {
            for (int c = 0; c < nch; ++c) barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// ST + Out, bf16, one workgroup per (sequence, head) and group of 16-row slices (the output pass's
// 8 value slices; the summary pass's 16, value and transition rows), for launches with many more
// slices than CUs. There every CU runs slice after slice, and what bounds a step is how many
// bytes each CU must pull from L2 per chunk: the per-slice kernel above loads the chunk's K, Q and
// factor record once per slice, this one once per group.
//  - Wavefronts 0..7 each run SPW slices' whole chunk step (one in the output pass, two in the
//    summary pass) with the states in registers, as the chunk algebra states it (no look-ahead, so
//    the key-key block of the record is not read): X = K S^T, Y = V - Gamma X,
//    R = T diag(beta) Y, O = scale Gamma Q S^T + P R, S <- Gamma_L S + K^T (e R). Each fragment of
//    the shared operands read from LDS feeds the wavefront's SPW slices.
//  - Wavefronts 8 and 9 move chunk c+1 (K and Q rows, T, coefficients, the eight V slices) into
//    the other of two LDS buffers with 16-byte direct loads while chunk c computes and, in the
//    summary pass, touch the lines of chunk c+2 so that those loads find them in L2.
//  - Wavefront 10 (output pass only) forms P_c = scale (D o Q_c K_c^T) from the K and Q rows in
//    LDS while the slice wavefronts form X, Y and R, once for the eight slices: Pre then neither
//    reads Q nor writes P, and the chain does not read P back.
// One workgroup barrier per chunk (two in the output pass: P_c is complete before the outputs).
// ---------------------------------------------------------------------------
template <int KD, bool SUMMARY>
struct HeadLds {
    typedef RowBlock<KD> RBk;
    static constexpr int KP = KD / 32, KB = KD / 16;
    static constexpr int SPW = SUMMARY ? 2 : 1;                        // slices per slice wavefront
    static constexpr int NCW = 8;                                      // slice wavefronts
    static constexpr int NS = NCW * SPW;                               // slices per workgroup
    static constexpr int NVS = 8;                                      // V slices held (V <= 128)
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

template <int KD, bool SUMMARY>
__global__ __launch_bounds__(SUMMARY ? 640 : 704) void gdn_chain_head_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const float* __restrict__ h0, const int32_t* __restrict__ cu, const int* __restrict__ chunk_off,
    const uint8_t* __restrict__ fac, int T, int H, int HK, int V, int n_seq, int nc, int ngrp,
    float scale, bf16_t* __restrict__ out, float* __restrict__ ht, float* __restrict__ Mout) {
    typedef HeadLds<KD, SUMMARY> SM;
    typedef RowBlock<KD> RBk;
    typedef Elem<bf16_t> El;
    constexpr int KP = SM::KP, KB = SM::KB, NS = SM::NS, SPW = SM::SPW, NCW = SM::NCW;
    constexpr int UST = (16 / RBk::RPB) * 1024;  // byte step of one 16-row token tile in a row block

    __shared__ __align__(16) uint8_t smem[SM::BYTES];
    typedef __attribute__((address_space(3))) uint8_t lds_u8;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    typedef __attribute__((address_space(3))) float lds_f32;
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
    const size_t rec_bytes = gdn_factor_bytes(2);
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
                if constexpr (!SUMMARY) {
                    barrier();  // P_c complete (wavefront 10)
                    // O^T = scale Gamma (S Q^T) + R^T P^T, token tile by token tile
                    const int t0 = bos + c * GC, L = min(GC, eos - t0);
                    i16x4 Rb[SPW][4];
#pragma unroll
                    for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
                        for (int ti = 0; ti < 4; ++ti) Rb[sl][ti] = El::pack(R[sl][ti]);
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt) {
                        f32x4 o[SPW];
#pragma unroll
                        for (int sl = 0; sl < SPW; ++sl) o[sl] = zero4();
#pragma unroll
                        for (int p = 0; p < KP; ++p) {
                            const bf16x8 qf = *(lds_bf16x8*)(B + SM::OFF_Q + orow[p] + tt * UST);
#pragma unroll
                            for (int sl = 0; sl < SPW; ++sl) o[sl] = mma32(cat8(Sf[sl][2 * p], Sf[sl][2 * p + 1]), qf, o[sl]);
                        }
                        const float gq = cf[16 * tt + ln] * scale;
#pragma unroll
                        for (int pp = 0; pp <= tt / 2; ++pp) {
                            const bf16x8 pf = *(lds_bf16x8*)(B + SM::OFF_P + tri_frag(tt, pp) * 1024 + lane * 16);
#pragma unroll
                            for (int sl = 0; sl < SPW; ++sl) o[sl] = mma32(cat8(Rb[sl][2 * pp], Rb[sl][2 * pp + 1]), pf, pp == 0 ? o[sl] * gq : o[sl]);
                        }
                        const int t = 16 * tt + ln;
                        pa[tt] = out + ((size_t)(b * T + t0 + t) * H + h) * V + row0 + 4 * lg;
                        pv[tt] = t < L;
#pragma unroll
                        for (int sl = 0; sl < SPW; ++sl) po[tt][sl] = El::pack(o[sl]);
                    }
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
                load_lds16(rec + 2 * GC * GC * 2, (uint8_t*)(B + SM::OFF_C));
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
                    const size_t off = r < 48 ? (size_t)r * 128 : (size_t)2 * GC * GC * 2 + (r - 48) * 128;
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
        // ================= P_c for the output pass: one wavefront =================
        // P^T tiles with K rows as A (rows s) and Q rows as B (columns t): the C tile holds, for lane
        // (ln, lg), P[16 ti + ln][16 tj + 4 lg + r], which is fragment (ti, tj / 2)'s lane content
        // (first or second half), the B operand that pairs with the R fragments of the same tokens.
        // The cumulative gates G are the coefficient block's last quarter.
        if constexpr (!SUMMARY) {
            int orow[KP];
#pragma unroll
            for (int p = 0; p < KP; ++p) orow[p] = RBk::off(ln, 4 * p + lg);
            barrier();
            for (int c = 0; c < nch; ++c) {
                lds_u8* B = buf(c);
                const lds_f32* cf = (const lds_f32*)(B + SM::OFF_C);
                bf16x8 kf[4][KP];
#pragma unroll
                for (int R = 0; R < 4; ++R)
#pragma unroll
                    for (int p = 0; p < KP; ++p) kf[R][p] = *(lds_bf16x8*)(B + SM::OFF_K + orow[p] + R * UST);
#pragma unroll
                for (int ti = 0; ti < 4; ++ti) {
                    bf16x8 qf[KP];
#pragma unroll
                    for (int p = 0; p < KP; ++p) qf[p] = *(lds_bf16x8*)(B + SM::OFF_Q + orow[p] + ti * UST);
                    const float Gt = cf[192 + 16 * ti + ln];
                    f32x4 PT[4];
#pragma unroll
                    for (int tj = 0; tj < 4; ++tj) {
                        PT[tj] = zero4();
                        if (tj <= ti) {
#pragma unroll
                            for (int p = 0; p < KP; ++p) PT[tj] = mma32(kf[tj][p], qf[p], PT[tj]);
                            const f32x4 Gs = *(const lds_f32x4*)(cf + 192 + 16 * tj + 4 * lg);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                // token s = 16 tj + 4 lg + r against t = 16 ti + ln: only s <= t, where G_t - G_s <= 0
                                const bool keep = tj < ti || 4 * lg + r <= ln;
                                PT[tj][r] = keep ? PT[tj][r] * (scale * __expf(fminf(Gt - Gs[r], 0.f))) : 0.f;
                            }
                        }
                    }
#pragma unroll
                    for (int p = 0; p <= ti / 2; ++p)
                        *(lds_bf16x8*)(B + SM::OFF_P + tri_frag(ti, p) * 1024 + lane * 16) = cat8(El::pack(PT[2 * p]), El::pack(PT[2 * p + 1]));
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                barrier();  // P_c complete
                barrier();  // end of the step
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

// The bf16 chain runs one workgroup per 16-row state slice (gdn_chain_1w_kernel) unless the launch
// has more than two slices per CU; then one workgroup per head (gdn_chain_head_kernel), which
// loads each chunk's shared operands once for all the head's slices.
bool gdn_chain_per_slice(long chains, int rows) { return chains * (rows / 16) <= 2L * device_cus(); }

template <typename ST, int KD>
static hipError_t run_gdn(int mode, const ST* q, const ST* k, const ST* v, const float* g,
                          const float* beta, const float* h0, const int32_t* cu,
                          const GdnWorkspace& ws, int N, int B, int T, int H, int HK, int V,
                          float scale, ST* out, float* ht, float* Mout, hipStream_t s, int stages, int pre_w,
                          const GateSrc& gs) {
    // the key-key block W and the decay-masked query-key block P are read only by the per-slice bf16
    // chain kernel (the per-head one forms P itself from the K and Q rows it holds)
    const int want_w = pre_w >= 0 ? pre_w : (gdn_chain_per_slice(N * H, mode == 0 ? V : V + KD) ? 1 : 0);
    const bool want_p = mode == 0 && gdn_chain_per_slice(N * H, V);
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
        if constexpr (sizeof(ST) == 2) {
            // When every unit fits on the GPU at once (8 two-wavefront workgroups per CU), the
            // chunk's latency is the launch's and two wavefronts per chunk halve it; otherwise one
            // wavefront per chunk spends fewer instructions per chunk.
            const unsigned gx = prep_grid(H, slots);
            const int2* tab = packed ? ws.table : nullptr;
            const bool two = (long)H * slots <= 8L * device_cus();
            if (two) {
                if (want_p)
                    gdn_prep_wave_kernel<KD, true, 2><<<gx, 128, 0, s>>>(q, k, g, beta, tab, cu, T, H, HK, nc, (int)slots, scale, ws.factors, want_w, gs);
                else
                    gdn_prep_wave_kernel<KD, false, 2><<<gx, 128, 0, s>>>(q, k, g, beta, tab, cu, T, H, HK, nc, (int)slots, scale, ws.factors, want_w, gs);
            } else {
                if (want_p)
                    gdn_prep_wave_kernel<KD, true, 1><<<gx, 64, 0, s>>>(q, k, g, beta, tab, cu, T, H, HK, nc, (int)slots, scale, ws.factors, want_w, gs);
                else
                    gdn_prep_wave_kernel<KD, false, 1><<<gx, 64, 0, s>>>(q, k, g, beta, tab, cu, T, H, HK, nc, (int)slots, scale, ws.factors, want_w, gs);
            }
        } else
            gdn_prep_kernel<ST, KD><<<dim3((unsigned)slots, H), 256, 0, s>>>(
                q, k, g, beta, packed ? ws.table : nullptr, cu, T, H, HK, nc, scale, mode == 0 ? 1 : 0,
                ws.factors, gs);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (!(stages & 2)) return hipSuccess;
    const int rows = mode == 0 ? V : V + KD;
    const int chains = N * H;
    if (chains == 0) return hipSuccess;
    if constexpr (sizeof(ST) == 2) {
        const int nvb = rows / 16;
        // more 16-row slices than two per CU: the CUs run slice after slice, and one workgroup per
        // head loads each chunk's shared operands once for all its slices
        if (!gdn_chain_per_slice(chains, rows)) {
            // slices per workgroup: the output pass's 8, the summary pass's 16 (all of a head's V + K rows)
            const int ns = mode == 0 ? HeadLds<KD, false>::NS : HeadLds<KD, true>::NS;
            const int ngrp = (nvb + ns - 1) / ns;
            const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * ngrp);
            if (mode == 0) {
                timing_begin("gdn_chain", s);
                gdn_chain_head_kernel<KD, false><<<grid, 704, 0, s>>>(
                    q, k, v, h0, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, ngrp, scale, out, ht, nullptr);
            } else {
                timing_begin("gdn_summary_chain", s);
                gdn_chain_head_kernel<KD, true><<<grid, 640, 0, s>>>(
                    q, k, v, nullptr, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, ngrp, scale, nullptr, ht, Mout);
            }
            timing_end(s);
            return hipGetLastError();
        }
        const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvb);
        if (mode == 0) {
            timing_begin("gdn_chain", s);
            gdn_chain_1w_kernel<KD, false><<<grid, 512, 0, s>>>(
                q, k, v, h0, cu, ws.chunk_off, ws.factors, T, H, HK, V, N, nc, nvb, scale, out, ht, nullptr);
        } else {
            timing_begin("gdn_summary_chain", s);
            gdn_chain_1w_kernel<KD, true><<<grid, 512, 0, s>>>(
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
                      float scale, void* out, float* ht, float* Mout, hipStream_t s, int stages, int pre_w,
                      const GateSrc* gate_src) {
    const GateSrc gs = gate_src ? *gate_src : GateSrc{nullptr, 0, nullptr, nullptr, 0, 0.f};
    if (bf16) {
        const bf16_t *qq = (const bf16_t*)q, *kk = (const bf16_t*)k, *vv = (const bf16_t*)v;
        if (K == 128) return run_gdn<bf16_t, 128>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (bf16_t*)out, ht, Mout, s, stages, pre_w, gs);
        return run_gdn<bf16_t, 64>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (bf16_t*)out, ht, Mout, s, stages, pre_w, gs);
    }
    const float *qq = (const float*)q, *kk = (const float*)k, *vv = (const float*)v;
    if (K == 128) return run_gdn<float, 128>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (float*)out, ht, Mout, s, stages, pre_w, gs);
    return run_gdn<float, 64>(mode, qq, kk, vv, g, beta, h0, cu, ws, N, B, T, H, HK, V, scale, (float*)out, ht, Mout, s, stages, pre_w, gs);
}

}  // namespace sf

// Gated Delta Rule chunk backward for gfx950: the gradients of the chunk forward with respect to q, k, v,
// the gate g, beta and the initial state, for upstream gradients of the outputs and the final states.
//
// The forward (attention-gym "Linear Attention", section "Gated Delta Rule", run per 64-token chunk with the
// StateFlow Section 2.2, Eq. (2) split) maps the entry state S of a chunk [V x K] to its exit state
//   S' = Gamma_L S + (diag(e) R)^T K,   R = T diag(beta) (V - diag(Gamma) K S^T),   T = (I + A)^-1,
//   O  = scale diag(Gamma) Q S^T + P R,  P = scale (D o Q K^T),  A = diag(beta) (D_strict o K K^T),
// with G the within-chunk cumulative gate, Gamma = exp(G), e = exp(G_L - G), D_ts = exp(G_t - G_s), s <= t.
// Its gradient runs the chain backwards (StateFlow Section 2.2, Eq. (6)-(7): the state gradient travels
// from the last chunk to the first): with dS' the gradient of the exit state,
//   dS = Gamma_L dS' - (dS' K^T) diag(e) W + dO^T Qt,   W = T diag(beta Gamma) K,   Qt = scale diag(Gamma) Q - P W,
// and, with the entry state S and dS' known, every input's gradient follows chunk by chunk:
//   dR = P^T dO + diag(e) K dS'^T,  dP = dO R^T,  dZ = T^T dR,  dT = dR Z^T  (Z = diag(beta) Y),
//   dY = diag(beta) dZ = dV,  dX = -diag(Gamma) dY,  dA = -T^T dT T^T (strictly lower part),
//   dQ = scale diag(Gamma) dO S + (scale D o dP) K,
//   dK = dX S + diag(e) R dS' + (scale D o dP)^T Q + F K + F^T K,  F = dA diag-row(beta) o D_strict,
//   dbeta = rowsum(Y o dZ) + rowsum(dA o D_strict o K K^T),
//   dG_t from the gate's four places (Gamma, e, D in P, D in A), dg = the reverse cumulative sum of dG.
//
// Kernels (float32 arithmetic throughout; q, k, v, do and the gradients dq, dk, dv in the input type):
//   gdn_bwd_prep_kernel    per (chunk, head): T, W, Qt and the coefficients into a record
//   gdn_bwd_states_kernel  per (sequence, head, 16-row slice): the forward chain, storing every chunk's
//                          entry state
//   gdn_bwd_dstate_kernel  per (sequence, head, 16-row slice): the reverse chain, storing every chunk's
//                          exit-state gradient, and dh0
//   gdn_bwd_grad_kernel    per (chunk, head): dq, dk, dv, dg, dbeta of the chunk
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {
namespace {

constexpr int BC = kGdnChunk;
constexpr int NT = 256;  // threads per workgroup of every backward kernel

// Record of one (chunk, head), floats: T [64][64] | W [64][KD] | Qt [64][KD] | coef [256]:
// [0,64) G, [64,128) Gamma, [128,192) e, [192,256) beta (padded tokens: g = beta = 0).
template <int KD>
struct BwdRec {
    static constexpr int T_OFF = 0, W_OFF = BC * BC, QT_OFF = W_OFF + BC * KD, C_OFF = QT_OFF + BC * KD;
    static constexpr int FLOATS = C_OFF + 256;
};

template <typename ST>
__device__ __forceinline__ float ld(const ST* p) { return Elem<ST>::to_f(*p); }

// element e of a 16-byte piece holding 8 bf16 or 4 float
template <typename ST>
__device__ __forceinline__ ST unit_of(const u128& u, int e) {
    if constexpr (sizeof(ST) == 2) {
        const uint32_t w = u[e >> 1];
        return (ST)((e & 1) ? (w >> 16) : (w & 0xffffu));
    } else {
        return __uint_as_float(u[e]);
    }
}

// A [ROWS][COLS] tile of ST (row stride ld elements; rows at or past rows_valid read as zero) moved to LDS as
// float [ROWS][COLS + 1] through registers in 16-byte pieces: load() puts every piece of the thread in flight
// at once, store() writes them to LDS, so a tile costs one load latency, and a chain can load the next
// chunk's tiles while it computes on the current ones.
template <typename ST, int ROWS, int COLS>
struct Tile {
    static constexpr int E = 16 / (int)sizeof(ST);
    static constexpr int PPR = COLS / E;                     // pieces per row
    static constexpr int PIECES = ROWS * PPR;
    static constexpr int PER = (PIECES + NT - 1) / NT;
    static_assert(COLS % E == 0, "tile rows are whole 16-byte pieces");
    u128 r[PER];
    __device__ __forceinline__ void load(const ST* __restrict__ base, long ld, int rows_valid) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = threadIdx.x + NT * p, row = idx / PPR, col = (idx % PPR) * E;
            r[p] = u128{0u, 0u, 0u, 0u};
            if (idx < PIECES && row < rows_valid) r[p] = *reinterpret_cast<const u128*>(base + row * ld + col);
        }
    }
    __device__ __forceinline__ void store(float* dst) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = threadIdx.x + NT * p, row = idx / PPR, col = (idx % PPR) * E;
            if (idx < PIECES)
#pragma unroll
                for (int e = 0; e < E; ++e) dst[row * (COLS + 1) + col + e] = Elem<ST>::to_f(unit_of<ST>(r[p], e));
        }
    }
};

// ---------------------------------------------------------------------------------------------------------
// Prep: per (chunk slot, head). G by a wave prefix sum, A and P from the raw products with the decay masks,
// T by forward substitution (one column per thread), then W and Qt.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_prep_kernel(const ST* __restrict__ q, const ST* __restrict__ k,
                                                          const float* __restrict__ g, const float* __restrict__ beta,
                                                          const int2* __restrict__ table, const int32_t* __restrict__ cu,
                                                          int T, int H, int nc, float scale, float* __restrict__ rec) {
    typedef BwdRec<KD> RL;
    constexpr int LK = KD + 1, LL = BC + 1;
    __shared__ float sK[BC * LK], sQ[BC * LK], sW[BC * LK];
    __shared__ float sA[BC * LL], sT[BC * LL], sP[BC * LL];
    __shared__ float sG[BC], sB[BC], sBG[BC];
    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const long row0 = (long)b * T + t0;
    {
        Tile<ST, BC, KD> tk, tq;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tq.load(q + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tk.store(sK);
        tq.store(sQ);
    }
    if (tid < BC) {
        const float gv = tid < L ? g[(row0 + tid) * H + h] : 0.f;
        const float bv = tid < L ? beta[(row0 + tid) * H + h] : 0.f;
        const float G = wave_inclusive_scan(gv);
        sB[tid] = bv;
        sG[tid] = G;
        sBG[tid] = bv * expf(G);
    }
    __syncthreads();
    // A = diag(beta) (D_strict o K K^T) and P = scale (D o Q K^T)
    for (int i = tid; i < BC * BC; i += NT) {
        const int t = i / BC, s = i % BC;
        float kk = 0.f, qk = 0.f;
        if (s <= t)
            for (int c = 0; c < KD; ++c) {
                kk += sK[t * LK + c] * sK[s * LK + c];
                qk += sQ[t * LK + c] * sK[s * LK + c];
            }
        const float d = s <= t ? expf(sG[t] - sG[s]) : 0.f;
        sA[t * LL + s] = s < t ? sB[t] * d * kk : 0.f;
        sP[t * LL + s] = scale * d * qk;
    }
    __syncthreads();
    if (tid < BC) {
        // column j = tid of T = (I + A)^-1 (unit lower triangular): x_j = 1, x_t = -sum_{j<=s<t} A_ts x_s
        const int j = tid;
        for (int t = 0; t < BC; ++t) {
            float x = t == j ? 1.f : 0.f;
            if (t > j)
                for (int s2 = j; s2 < t; ++s2) x -= sA[t * LL + s2] * sT[s2 * LL + j];
            sT[t * LL + j] = x;
        }
    }
    __syncthreads();
    float* R = rec + ((size_t)slot * H + h) * RL::FLOATS;
    // W[t][c] = sum_{s<=t} T[t][s] beta_s Gamma_s K[s][c]; thread owns row t = tid / 4, columns tid % 4 + 4 m
    const int t = tid >> 2;
    for (int m = 0; m < KD / 4; ++m) {
        const int c = (tid & 3) + 4 * m;
        float w = 0.f;
        for (int s2 = 0; s2 <= t; ++s2) w += sT[t * LL + s2] * sBG[s2] * sK[s2 * LK + c];
        sW[t * LK + c] = w;
        R[RL::W_OFF + t * KD + c] = w;
    }
    __syncthreads();
    // Qt[t][c] = scale Gamma_t Q[t][c] - sum_{s<=t} P[t][s] W[s][c]
    const float gq = scale * expf(sG[t]);
    for (int m = 0; m < KD / 4; ++m) {
        const int c = (tid & 3) + 4 * m;
        float acc = 0.f;
        for (int s2 = 0; s2 <= t; ++s2) acc += sP[t * LL + s2] * sW[s2 * LK + c];
        R[RL::QT_OFF + t * KD + c] = gq * sQ[t * LK + c] - acc;
    }
    for (int i = tid; i < BC * BC; i += NT) R[RL::T_OFF + i] = sT[(i / BC) * LL + i % BC];
    if (tid < BC) {
        const float G = sG[tid], GL = sG[BC - 1];
        R[RL::C_OFF + tid] = G;
        R[RL::C_OFF + 64 + tid] = expf(G);
        R[RL::C_OFF + 128 + tid] = expf(GL - G);
        R[RL::C_OFF + 192 + tid] = sB[tid];
    }
}

// Sequence n of a (sequence, head) chain: batch row, token range, first chunk slot.
__device__ __forceinline__ void seq_of(int n, const int32_t* cu, const int* chunk_off, int T, int nc, int& b,
                                       int& bos, int& eos, int& slot0) {
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
}

// ---------------------------------------------------------------------------------------------------------
// States: the forward chain of one 16-row slice of one (sequence, head), storing the entry state of every
// chunk (float32 [slot][H][V][K]). Thread owns state entries e = tid + 256 m (row e / KD, column e % KD).
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_states_kernel(const ST* __restrict__ k, const ST* __restrict__ v,
                                                            const float* __restrict__ h0, const int32_t* __restrict__ cu,
                                                            const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                            int T, int H, int V, int n_seq, int nc, int nvs,
                                                            float* __restrict__ states) {
    typedef BwdRec<KD> RL;
    constexpr int LK = KD + 1, LL = BC + 1, LV = 17, NE = 16 * KD / NT;
    __shared__ float sK[BC * LK], sS[16 * LK], sT[BC * LL], sV[BC * LV], sZ[BC * LV], sC[256];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
    int b, bos, eos, slot0;
    seq_of(n, cu, chunk_off, T, nc, b, bos, eos, slot0);
    const int nch = (eos - bos + BC - 1) / BC;
    float S[NE];
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + NT * m, r = e / KD, c = e % KD;
        S[m] = h0 ? h0[(((size_t)n * H + h) * V + v0 + r) * KD + c] : 0.f;
    }
    const int t = tid >> 2, v4 = (tid & 3) * 4;
    // chunk ci's K rows, T, coefficients and V slice, loaded one chunk ahead
    Tile<ST, BC, KD> tk;
    Tile<float, BC, BC> tt;
    Tile<ST, BC, 16> tv;
    float cf = 0.f;
    auto issue = [&](int ci) __attribute__((always_inline)) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
        const float* R = rec + ((size_t)(slot0 + ci) * H + h) * RL::FLOATS;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tt.load(R + RL::T_OFF, BC, BC);
        tv.load(v + (row0 * H + h) * (long)V + v0, (long)H * V, L);
        cf = R[RL::C_OFF + tid];
    };
    if (nch > 0) issue(0);
    for (int ci = 0; ci < nch; ++ci) {
        float* Sout = states + (((size_t)(slot0 + ci) * H + h) * V + v0) * KD;
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + NT * m;
            Sout[(e / KD) * KD + e % KD] = S[m];
            sS[(e / KD) * LK + e % KD] = S[m];
        }
        tk.store(sK);
        tt.store(sT);
        tv.store(sV);
        sC[tid] = cf;
        __syncthreads();
        if (ci + 1 < nch) issue(ci + 1);
        // Z = diag(beta) (V - diag(Gamma) K S^T) on (token t, values v4 .. v4 + 3)
        {
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < KD; ++c) {
                const float kt = sK[t * LK + c];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] += kt * sS[(v4 + j) * LK + c];
            }
            const float gam = sC[64 + t], bt = sC[192 + t];
#pragma unroll
            for (int j = 0; j < 4; ++j) sZ[t * LV + v4 + j] = bt * (sV[t * LV + v4 + j] - gam * x[j]);
        }
        __syncthreads();
        // e R = e T Z (into sV, no longer needed)
        {
            float r[4] = {0.f, 0.f, 0.f, 0.f};
            for (int s2 = 0; s2 <= t; ++s2) {
                const float ts = sT[t * LL + s2];
#pragma unroll
                for (int j = 0; j < 4; ++j) r[j] += ts * sZ[s2 * LV + v4 + j];
            }
            const float et = sC[128 + t];
#pragma unroll
            for (int j = 0; j < 4; ++j) sV[t * LV + v4 + j] = et * r[j];
        }
        __syncthreads();
        // S <- Gamma_L S + (e R)^T K
        const float gl = sC[64 + BC - 1];
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + NT * m, r = e / KD, c = e % KD;
            float acc = gl * S[m];
            for (int tt = 0; tt < BC; ++tt) acc += sV[tt * LV + r] * sK[tt * LK + c];
            S[m] = acc;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------------------
// Reverse chain: one 16-row slice of one (sequence, head), from dht (or zero) backwards. Before chunk c's
// step the slice holds the gradient of chunk c's exit state, stored as float32 [slot][H][V][K]; after chunk
// 0 it is dh0.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_dstate_kernel(const ST* __restrict__ k, const ST* __restrict__ dout,
                                                            const float* __restrict__ dht, const int32_t* __restrict__ cu,
                                                            const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                            int T, int H, int V, int n_seq, int nc, int nvs,
                                                            float* __restrict__ dstates, float* __restrict__ dh0) {
    typedef BwdRec<KD> RL;
    constexpr int LK = KD + 1, LV = 17, NE = 16 * KD / NT, LZ = BC + 1;
    __shared__ float sK[BC * LK], sW[BC * LK], sQt[BC * LK], sD[16 * LK], sO[BC * LV], sZ[16 * LZ], sC[256];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
    int b, bos, eos, slot0;
    seq_of(n, cu, chunk_off, T, nc, b, bos, eos, slot0);
    const int nch = (eos - bos + BC - 1) / BC;
    float dS[NE];
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + NT * m;
        dS[m] = dht ? dht[(((size_t)n * H + h) * V + v0 + e / KD) * KD + e % KD] : 0.f;
    }
    // chunk ci's K rows, W, Qt, coefficients and dO slice, loaded one chunk ahead (chunks run backwards)
    Tile<ST, BC, KD> tk;
    Tile<float, BC, KD> tw, tq;
    Tile<ST, BC, 16> to;
    float cf = 0.f;
    auto issue = [&](int ci) __attribute__((always_inline)) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
        const float* R = rec + ((size_t)(slot0 + ci) * H + h) * RL::FLOATS;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tw.load(R + RL::W_OFF, KD, BC);
        tq.load(R + RL::QT_OFF, KD, BC);
        to.load(dout + (row0 * H + h) * (long)V + v0, (long)H * V, L);
        cf = R[RL::C_OFF + tid];
    };
    if (nch > 0) issue(nch - 1);
    for (int ci = nch - 1; ci >= 0; --ci) {
        float* Dout = dstates + (((size_t)(slot0 + ci) * H + h) * V + v0) * KD;
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + NT * m;
            Dout[(e / KD) * KD + e % KD] = dS[m];
            sD[(e / KD) * LK + e % KD] = dS[m];
        }
        tk.store(sK);
        tw.store(sW);
        tq.store(sQt);
        to.store(sO);
        sC[tid] = cf;
        __syncthreads();
        if (ci > 0) issue(ci - 1);
        // Z[r][t] = e_t (dS' K^T)[r][t]; thread: row r = tid / 16, tokens 4 (tid % 16) .. + 3
        {
            const int r = tid >> 4, t4 = (tid & 15) * 4;
            float z[4] = {0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < KD; ++c) {
                const float d = sD[r * LK + c];
#pragma unroll
                for (int j = 0; j < 4; ++j) z[j] += d * sK[(t4 + j) * LK + c];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) sZ[r * LZ + t4 + j] = sC[128 + t4 + j] * z[j];
        }
        __syncthreads();
        // dS = Gamma_L dS' - Z W + dO^T Qt
        const float gl = sC[64 + BC - 1];
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + NT * m, r = e / KD, c = e % KD;
            float acc = gl * dS[m];
            for (int tt = 0; tt < BC; ++tt) acc += sO[tt * LV + r] * sQt[tt * LK + c] - sZ[r * LZ + tt] * sW[tt * LK + c];
            dS[m] = acc;
        }
        __syncthreads();
    }
    if (dh0) {
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + NT * m;
            dh0[(((size_t)n * H + h) * V + v0 + e / KD) * KD + e % KD] = dS[m];
        }
    }
}

// ---------------------------------------------------------------------------------------------------------
// Gradients of one (chunk slot, head): the value dimension in 16-row slices (entry state, exit-state
// gradient, dO and V of the slice), dP, dT, dq and dk accumulated over the slices in registers, then the
// solve and gate terms. Thread ownership: token t = tid / 4 of every [64 x 16] slice matrix (values
// v4 .. v4 + 3, v4 = 4 (tid % 4)), of dP and dT (columns tid % 4 + 4 j) and of dq, dk (columns
// tid % 4 + 4 m).
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_grad_kernel(
    const ST* __restrict__ q, const ST* __restrict__ k, const ST* __restrict__ v, const ST* __restrict__ dout,
    const float* __restrict__ rec, const float* __restrict__ states, const float* __restrict__ dstates,
    const int2* __restrict__ table, const int32_t* __restrict__ cu, int T, int H, int V, int nc, float scale,
    ST* __restrict__ dq, ST* __restrict__ dk, ST* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta) {
    typedef BwdRec<KD> RL;
    constexpr int LK = KD + 1, LL = BC + 1, LV = 17, NM = KD / 4;
    __shared__ float sK[BC * LK], sQ[BC * LK], sT[BC * LL], sQK[BC * LL], sKK[BC * LL], sC[256];
    // per-slice region; after the slices it holds dP | dT (two [64][65] blocks)
    constexpr int SLICE_FLOATS = 2 * 16 * LK + 4 * BC * LV > 2 * BC * LL ? 2 * 16 * LK + 4 * BC * LV : 2 * BC * LL;
    __shared__ float sX[SLICE_FLOATS];
    float* const sS = sX;                 // [16][LK] entry state of the slice
    float* const sD = sX + 16 * LK;       // [16][LK] exit-state gradient of the slice
    float* const sO = sX + 32 * LK;       // [64][LV] dO of the slice
    float* const sZ = sO + BC * LV;       // [64][LV] Z = diag(beta) Y
    float* const sR = sZ + BC * LV;       // [64][LV] R
    float* const sdR = sR + BC * LV;      // [64][LV] dR, later dX
    float* const sdP = sX;                // [64][LL] after the slices
    float* const sdT = sX + BC * LL;      // [64][LL] after the slices
    __shared__ float sDG[BC];

    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const long row0 = (long)b * T + t0;
    const float* Rc = rec + ((size_t)slot * H + h) * RL::FLOATS;
    {
        Tile<ST, BC, KD> tk, tq;
        Tile<float, BC, BC> tt;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tq.load(q + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tt.load(Rc + RL::T_OFF, BC, BC);
        sC[tid] = Rc[RL::C_OFF + tid];
        tk.store(sK);
        tq.store(sQ);
        tt.store(sT);
    }
    __syncthreads();
    const int t = tid >> 2, q4 = tid & 3, v4 = 4 * q4;
    // raw Q K^T and K K^T on the thread's (t, s) entries
    for (int j = 0; j < 16; ++j) {
        const int s2 = q4 + 4 * j;
        float qk = 0.f, kk = 0.f;
        for (int c = 0; c < KD; ++c) {
            qk += sQ[t * LK + c] * sK[s2 * LK + c];
            kk += sK[t * LK + c] * sK[s2 * LK + c];
        }
        sQK[t * LL + s2] = qk;
        sKK[t * LL + s2] = kk;
    }
    const float Gt = sC[t], gamt = sC[64 + t], et = sC[128 + t], bt = sC[192 + t], gl = sC[64 + BC - 1];
    float aP[16], aT[16], aQ[NM], aK[NM];
#pragma unroll
    for (int j = 0; j < 16; ++j) aP[j] = aT[j] = 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m) aQ[m] = aK[m] = 0.f;
    float pGam = 0.f, pE = 0.f, pB = 0.f, pGL = 0.f;  // partial sums of dGamma_t, de_t, dbeta_t, dGamma_L
    const int nvs = V / 16;
    __syncthreads();
    // the slice's entry state, exit-state gradient and dO, loaded one slice ahead
    Tile<float, 16, KD> ts, td;
    Tile<ST, BC, 16> to;
    auto issue = [&](int vs) __attribute__((always_inline)) {
        const int v0 = 16 * vs;
        ts.load(states + (((size_t)slot * H + h) * V + v0) * KD, KD, 16);
        td.load(dstates + (((size_t)slot * H + h) * V + v0) * KD, KD, 16);
        to.load(dout + (row0 * H + h) * (long)V + v0, (long)H * V, L);
    };
    issue(0);
    for (int vs = 0; vs < nvs; ++vs) {
        const int v0 = 16 * vs;
        ts.store(sS);
        td.store(sD);
        to.store(sO);
        if (vs + 1 < nvs) issue(vs + 1);
        float vv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) vv[j] = t < L ? ld(v + ((row0 + t) * H + h) * (long)V + v0 + v4 + j) : 0.f;
        __syncthreads();
        // X = K S^T, QS = Q S^T, KdS = K dS'^T on (t, v4 .. v4 + 3)
        float X[4] = {0.f, 0.f, 0.f, 0.f}, QS[4] = {0.f, 0.f, 0.f, 0.f}, KdS[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < KD; ++c) {
            const float kt = sK[t * LK + c], qt = sQ[t * LK + c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sv = sS[(v4 + j) * LK + c], dv_ = sD[(v4 + j) * LK + c];
                X[j] += kt * sv;
                QS[j] += qt * sv;
                KdS[j] += kt * dv_;
            }
        }
        float Y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Y[j] = vv[j] - gamt * X[j];
            sZ[t * LV + v4 + j] = bt * Y[j];
            pGam += scale * sO[t * LV + v4 + j] * QS[j];
        }
        __syncthreads();
        // R = T Z;  dR = P^T dO + e KdS with P[s][t] = scale exp(G_s - G_t) QK[s][t], s >= t
        float Rv[4] = {0.f, 0.f, 0.f, 0.f}, dR[4];
        for (int s2 = 0; s2 <= t; ++s2) {
            const float ts = sT[t * LL + s2];
#pragma unroll
            for (int j = 0; j < 4; ++j) Rv[j] += ts * sZ[s2 * LV + v4 + j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dR[j] = et * KdS[j];
        for (int s2 = t; s2 < BC; ++s2) {
            const float p = scale * expf(sC[s2] - Gt) * sQK[s2 * LL + t];
#pragma unroll
            for (int j = 0; j < 4; ++j) dR[j] += p * sO[s2 * LV + v4 + j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sR[t * LV + v4 + j] = Rv[j];
            sdR[t * LV + v4 + j] = dR[j];
            pE += Rv[j] * KdS[j];
        }
        __syncthreads();
        // dZ = T^T dR; dbeta, dY = dV, dX = -Gamma dY; dP += dO R^T, dT += dR Z^T on the thread's entries
        float dZ[4] = {0.f, 0.f, 0.f, 0.f};
        for (int s2 = t; s2 < BC; ++s2) {
            const float ts = sT[s2 * LL + t];
#pragma unroll
            for (int j = 0; j < 4; ++j) dZ[j] += ts * sdR[s2 * LV + v4 + j];
        }
#pragma unroll 1
        for (int vv2 = 0; vv2 < 16; ++vv2) {
            const float o = sO[t * LV + vv2], r = sdR[t * LV + vv2];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int s2 = q4 + 4 * j;
                aP[j] += o * sR[s2 * LV + vv2];
                aT[j] += r * sZ[s2 * LV + vv2];
            }
        }
        float dX[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pB += Y[j] * dZ[j];
            const float dY = bt * dZ[j];
            if (t < L) dv[((row0 + t) * H + h) * (long)V + v0 + v4 + j] = Elem<ST>::from_f(dY);
            dX[j] = -gamt * dY;
            pGam -= dY * X[j];
        }
        for (int i = tid; i < 16 * KD; i += NT) pGL += sS[(i / KD) * LK + i % KD] * sD[(i / KD) * LK + i % KD];
        __syncthreads();  // every read of dR is done: it becomes dX
#pragma unroll
        for (int j = 0; j < 4; ++j) sdR[t * LV + v4 + j] = dX[j];
        __syncthreads();
        // dq += scale Gamma_t dO S;  dk += dX S + e R dS'
#pragma unroll 1
        for (int vv2 = 0; vv2 < 16; ++vv2) {
            const float o = scale * gamt * sO[t * LV + vv2], x = sdR[t * LV + vv2], r = et * sR[t * LV + vv2];
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int c = q4 + 4 * m;
                const float sv = sS[vv2 * LK + c];
                aQ[m] += o * sv;
                aK[m] += x * sv + r * sD[vv2 * LK + c];
            }
        }
        __syncthreads();
    }
    // dP and dT to LDS; U = dT T^T on the thread's entries (T lower: j <= s)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int s2 = q4 + 4 * j;
        sdP[t * LL + s2] = aP[j];
        sdT[t * LL + s2] = aT[j];
    }
    __syncthreads();
    float U[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int s2 = q4 + 4 * j;
        float u = 0.f;
        for (int jj = 0; jj <= s2; ++jj) u += sdT[t * LL + jj] * sT[s2 * LL + jj];
        U[j] = u;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) sdT[t * LL + q4 + 4 * j] = U[j];
    __syncthreads();
    // dA[t][s] = -sum_{j >= t} T[j][t] U[j][s] for s < t; then the gate terms, F and (scale D o dP)
    float rowc = 0.f;
    float Fv[16], DP[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int s2 = q4 + 4 * j;
        float dA = 0.f;
        if (s2 < t)
            for (int jj = t; jj < BC; ++jj) dA -= sT[jj * LL + t] * sdT[jj * LL + s2];
        const float d = s2 <= t ? expf(Gt - sC[s2]) : 0.f;
        const float kk = sKK[t * LL + s2];
        pB += dA * d * kk;                       // (dA is zero unless s < t)
        Fv[j] = dA * bt * d;
        DP[j] = s2 <= t ? scale * d * aP[j] : 0.f;
        const float c = DP[j] * sQK[t * LL + s2] + Fv[j] * kk;
        rowc += c;
        sKK[t * LL + s2] = c;                    // own entry: K K^T is not read again
    }
    __syncthreads();
    // (scale D o dP) into sdP, F into sdT (own entries; U is no longer read)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        sdP[t * LL + q4 + 4 * j] = DP[j];
        sdT[t * LL + q4 + 4 * j] = Fv[j];
    }
    __syncthreads();
    // dq += (scale D o dP) K;  dk += (scale D o dP)^T Q + F K + F^T K
#pragma unroll 1
    for (int s2 = 0; s2 < BC; ++s2) {
        const float p = sdP[t * LL + s2], pt = sdP[s2 * LL + t], f = sdT[t * LL + s2] + sdT[s2 * LL + t];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int c = q4 + 4 * m;
            const float ks = sK[s2 * LK + c];
            aQ[m] += p * ks;
            aK[m] += pt * sQ[s2 * LK + c] + f * ks;
        }
    }
    // the four threads of token t hold quarters of its row sums
#pragma unroll
    for (int o = 1; o <= 2; o <<= 1) {
        pGam += __shfl_xor(pGam, o, 64);
        pE += __shfl_xor(pE, o, 64);
        pB += __shfl_xor(pB, o, 64);
        rowc += __shfl_xor(rowc, o, 64);
    }
    // <dS', S> over the workgroup
    for (int o = 1; o < 64; o <<= 1) pGL += __shfl_xor(pGL, o, 64);
    __shared__ float sRed[NT / 64], sEE[BC];
    if ((tid & 63) == 0) sRed[tid >> 6] = pGL;
    // dG_t = dGamma_t Gamma_t - de_t e_t + (row sum - column sum of the gate terms of D)
    if (q4 == 0) {
        sDG[t] = pGam * gamt - pE * et + rowc;
        sEE[t] = pE * et;
    }
    if (t < L) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int c = q4 + 4 * m;
            dq[((row0 + t) * H + h) * (long)KD + c] = Elem<ST>::from_f(aQ[m]);
            dk[((row0 + t) * H + h) * (long)KD + c] = Elem<ST>::from_f(aK[m]);
        }
        if (q4 == 0) dbeta[(row0 + t) * H + h] = pB;
    }
    __syncthreads();
    if (tid < BC) {
        float col = 0.f;
        for (int tt = 0; tt < BC; ++tt) col += sKK[tt * LL + tid];
        float dG = sDG[tid] - col;
        if (tid == BC - 1) {
            // G_L (token 63: padded tokens repeat the last real G) also carries e's and Gamma_L's terms
            float se = 0.f;
            for (int tt = 0; tt < BC; ++tt) se += sEE[tt];
            float gsum = 0.f;
#pragma unroll
            for (int w = 0; w < NT / 64; ++w) gsum += sRed[w];
            dG += se + gsum * gl;
        }
        // dg = the reverse cumulative sum of dG over the chunk: lane l scans dG of token 63 - l
        const float rev = __shfl(dG, BC - 1 - tid, 64);
        const float cs = wave_inclusive_scan(rev);
        const float dgt = __shfl(cs, BC - 1 - tid, 64);
        if (tid < L) dg[(row0 + tid) * H + h] = dgt;
    }
}

template <typename ST, int KD>
hipError_t run_bwd(const ST* q, const ST* k, const ST* v, const float* g, const float* beta, const float* h0,
                   const ST* dout, const float* dht, const int32_t* cu, const GdnBwdWorkspace& ws, int N, int B,
                   int T, int H, int V, float scale, ST* dq, ST* dk, ST* dv, float* dg, float* dbeta, float* dh0,
                   hipStream_t s) {
    const bool packed = cu != nullptr;
    const long slots = gdn_slots(B, T, N, packed);
    const int nc = (T + BC - 1) / BC;
    hipError_t err;
    if (packed) {
        err = launch_chunk_table(cu, N, BC, slots, ws.chunk_off, ws.table, s);
        if (err != hipSuccess) return err;
    }
    const int2* table = packed ? ws.table : nullptr;
    if (slots > 0) {
        timing_begin("gdn_bwd_prep", s);
        gdn_bwd_prep_kernel<ST, KD><<<dim3((unsigned)slots, H), NT, 0, s>>>(q, k, g, beta, table, cu, T, H, nc, scale, ws.rec);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const long chains = (long)N * H;
    if (chains > 0) {
        const int nvs = V / 16;
        const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvs);
        timing_begin("gdn_bwd_states", s);
        gdn_bwd_states_kernel<ST, KD><<<grid, NT, 0, s>>>(k, v, h0, cu, ws.chunk_off, ws.rec, T, H, V, N, nc, nvs, ws.states);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        timing_begin("gdn_bwd_dstate", s);
        gdn_bwd_dstate_kernel<ST, KD><<<grid, NT, 0, s>>>(k, dout, dht, cu, ws.chunk_off, ws.rec, T, H, V, N, nc, nvs,
                                                          ws.dstates, dh0);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (slots > 0) {
        timing_begin("gdn_bwd_grad", s);
        gdn_bwd_grad_kernel<ST, KD><<<dim3((unsigned)slots, H), NT, 0, s>>>(q, k, v, dout, ws.rec, ws.states, ws.dstates,
                                                                          table, cu, T, H, V, nc, scale, dq, dk, dv, dg,
                                                                          dbeta);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gdn_bwd(bool bf16, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* h0, const void* dout, const float* dht,
                          const int32_t* cu, const GdnBwdWorkspace& ws, int N, int B, int T, int H, int K,
                          int V, float scale, void* dq, void* dk, void* dv, float* dg, float* dbeta,
                          float* dh0, hipStream_t s) {
    if (bf16) {
        typedef bf16_t E;
        auto c = [](const void* x) { return static_cast<const E*>(x); };
        auto m = [](void* x) { return static_cast<E*>(x); };
        if (K == 128)
            return run_bwd<E, 128>(c(q), c(k), c(v), g, beta, h0, c(dout), dht, cu, ws, N, B, T, H, V, scale, m(dq), m(dk),
                                   m(dv), dg, dbeta, dh0, s);
        return run_bwd<E, 64>(c(q), c(k), c(v), g, beta, h0, c(dout), dht, cu, ws, N, B, T, H, V, scale, m(dq), m(dk),
                              m(dv), dg, dbeta, dh0, s);
    }
    typedef float E;
    auto c = [](const void* x) { return static_cast<const E*>(x); };
    auto m = [](void* x) { return static_cast<E*>(x); };
    if (K == 128)
        return run_bwd<E, 128>(c(q), c(k), c(v), g, beta, h0, c(dout), dht, cu, ws, N, B, T, H, V, scale, m(dq), m(dk),
                               m(dv), dg, dbeta, dh0, s);
    return run_bwd<E, 64>(c(q), c(k), c(v), g, beta, h0, c(dout), dht, cu, ws, N, B, T, H, V, scale, m(dq), m(dk), m(dv),
                          dg, dbeta, dh0, s);
}

}  // namespace sf

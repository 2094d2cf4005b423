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
// Kernels (float32 accumulation and elementwise arithmetic; q, k, v, do and the gradients dq, dk, dv in the
// input type; the products in the input type's arithmetic):
//   gdn_bwd_prep_kernel    per (chunk, head): T, W, Qt and the coefficients into a record
//                          (gdn_bwd_prep16_kernel for bf16 inputs)
//   gdn_bwd_states_kernel  per (sequence, head, 16-row slice): the forward chain, storing every chunk's
//                          entry state (gdn_bwd_states16_kernel for bf16 inputs)
//   gdn_bwd_dstate_kernel  per (sequence, head, 16-row slice): the reverse chain, storing every chunk's
//                          exit-state gradient, and dh0 (gdn_bwd_dstate16_kernel for bf16 inputs)
//   gdn_bwd_grad_kernel    per (chunk, head): dq, dk, dv, dg, dbeta of the chunk (gdn_bwd_grad16_kernel for
//                          bf16 inputs)
// The float32-input kernels keep their operands in float32 in LDS; the bf16 ones keep bf16 operands and
// read them in the row and column forms described at gdn_bwd_grad16_kernel. The bf16 prep, gradient and
// state-gradient kernels run eight wavefronts, two per 16-token tile (or per key tile pair).
#include <type_traits>

#include "f32_tiles.h"
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {
namespace {

constexpr int BC = kGdnChunk;
constexpr int NT = f32t::NT;  // threads per workgroup of every backward kernel

// Record of one (chunk, head), floats: T [64][64] | W [64][KD] | Qt [64][KD] | coef [256]:
// [0,64) G, [64,128) Gamma, [128,192) e, [192,256) beta (padded tokens: g = beta = 0).
template <int KD>
struct BwdRec {
    static constexpr int T_OFF = 0, W_OFF = BC * BC, QT_OFF = W_OFF + BC * KD, C_OFF = QT_OFF + BC * KD;
    static constexpr int FLOATS = C_OFF + 256;
};
// T, W and Qt are stored in the input type at their offsets (for bf16 inputs half of each region): they enter
// only products, whose tiles round their operands to the input type in any case (unscaled).
template <typename ST, int KD>
__device__ __forceinline__ ST* rec_t(float* R) { return reinterpret_cast<ST*>(R + BwdRec<KD>::T_OFF); }
template <typename ST, int KD>
__device__ __forceinline__ const ST* rec_t(const float* R) { return reinterpret_cast<const ST*>(R + BwdRec<KD>::T_OFF); }
template <typename ST, int KD>
__device__ __forceinline__ ST* rec_w(float* R) { return reinterpret_cast<ST*>(R + BwdRec<KD>::W_OFF); }
template <typename ST, int KD>
__device__ __forceinline__ ST* rec_qt(float* R) { return reinterpret_cast<ST*>(R + BwdRec<KD>::QT_OFF); }
template <typename ST, int KD>
__device__ __forceinline__ const ST* rec_w(const float* R) { return reinterpret_cast<const ST*>(R + BwdRec<KD>::W_OFF); }
template <typename ST, int KD>
__device__ __forceinline__ const ST* rec_qt(const float* R) { return reinterpret_cast<const ST*>(R + BwdRec<KD>::QT_OFF); }

template <typename ST>
__device__ __forceinline__ float ld(const ST* p) { return Elem<ST>::to_f(*p); }

using f32t::Tile;
using f32t::mm4;
using f32t::mmb;
using f32t::mmg;
using f32t::mmx;
using f32t::unit_of;

// ---------------------------------------------------------------------------------------------------------
// Prep: per (chunk slot, head), on float32 MFMA tiles (wavefront w owns token rows 16 w .. 16 w + 15). G by a wave
// prefix sum; A and P from the raw products with the decay masks; T by 16x16 blocks (the four diagonal blocks by
// column substitution, one wavefront each, then T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj block diagonal by block
// diagonal); then W = T diag(beta Gamma) K and Qt = scale Gamma Q - P W.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_prep_kernel(const ST* __restrict__ q, const ST* __restrict__ k,
                                                          const float* __restrict__ g, const float* __restrict__ beta,
                                                          const int2* __restrict__ table, const int32_t* __restrict__ cu,
                                                          int T, int H, int nc, float scale, float* __restrict__ rec) {
    typedef BwdRec<KD> RL;
    // K, Q and W in LDS in the input type (bf16 rows of 16-byte pieces: the products read them as they are, the
    // same bf16 values the float32 tiles would round them to)
    constexpr bool B16 = sizeof(ST) == 2;
    typedef typename std::conditional<B16, bf16_t, float>::type LT;
    constexpr int LK = B16 ? KD + 8 : KD + 1, LL = BC + 1, LU = 17, NJ = KD / 16;
    __shared__ __align__(16) LT sK[BC * LK], sQ[BC * LK], sW[BC * LK];
    __shared__ float sA[BC * LL], sT[BC * LL], sP[BC * LL];
    __shared__ float sG[BC], sB[BC], sGam[BC], sU[4 * 16 * LU];
    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const long row0 = (long)b * T + t0;
    {
        Tile<ST, BC, KD> tk, tq;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tq.load(q + (row0 * H + h) * (long)KD, (long)H * KD, L);
        if constexpr (B16) {
            tk.template store_raw<LK>(sK);
            tq.template store_raw<LK>(sQ);
        } else {
            tk.store(sK);
            tq.store(sQ);
        }
    }
    if (tid < BC) {
        const float gv = tid < L ? g[(row0 + tid) * H + h] : 0.f;
        sB[tid] = tid < L ? beta[(row0 + tid) * H + h] : 0.f;
        const float G = wave_inclusive_scan(gv);
        sG[tid] = G;
        sGam[tid] = expf(G);
    }
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    int tr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) tr[r] = 16 * w + 4 * lg + r;
    // A = diag(beta) (D_strict o K K^T) and P = scale (D o Q K^T) on the wavefront's row tile
    for (int j = 0; j < 4; ++j) {
        f32x4 kk = zero4(), qk = zero4();
        if (j <= w) {
            if constexpr (B16) {
                kk = mmb(sK + 16 * w * LK, LK, sK + 16 * j * LK, LK, 0, KD, kk);
                qk = mmb(sQ + 16 * w * LK, LK, sK + 16 * j * LK, LK, 0, KD, qk);
            } else {
                kk = mmx<ST>(sK + 16 * w * LK, LK, 1, sK + 16 * j * LK, 1, LK, 0, KD, kk);
                qk = mmx<ST>(sQ + 16 * w * LK, LK, 1, sK + 16 * j * LK, 1, LK, 0, KD, qk);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tr[r], s2 = 16 * j + ln;
            const float d = s2 <= t ? expf(sG[t] - sG[s2]) : 0.f;
            sA[t * LL + s2] = s2 < t ? sB[t] * d * kk[r] : 0.f;
            sP[t * LL + s2] = scale * d * qk[r];
            sT[t * LL + s2] = 0.f;
        }
    }
    __syncthreads();
    // diagonal blocks: wavefront w inverts block w, lane j < 16 solving column j: x_j = 1,
    // x_i = -sum_{j<=s<i} A_ii[i][s] x_s
    // (the column in registers; its entries above the diagonal are zero, so the terms s2 < j change nothing)
    if (lane < 16) {
        const int o = 16 * w, j = lane;
        float xs[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = i == j ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < i; ++s2) x -= sA[(o + i) * LL + o + s2] * xs[s2];
            xs[i] = x;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(o + i) * LL + o + j] = xs[i];
    }
    // (K scaled by beta Gamma per token, for W: K is not read again as itself)
    for (int i = tid; i < BC * KD; i += NT) {
        const int t = i / KD, c = i % KD;
        sK[t * LK + c] = Elem<ST>::from_f(Elem<ST>::to_f(sK[t * LK + c]) * (sB[t] * sGam[t]));
    }
    __syncthreads();
    // off-diagonal blocks, one block diagonal dd at a time: block (i, j = i - dd) by wavefront i
    for (int dd = 1; dd < 4; ++dd) {
        const int i = w, j = w - dd;
        if (j >= 0) {
            // U = sum_{kb=j}^{i-1} A_i,kb T_kb,j (16 x 16, k over the tokens of blocks j .. i-1)
            const f32x4 Uv = mm4(sA + 16 * i * LL + 16 * j, LL, 1, sT + 16 * j * LL + 16 * j, LL, 1, 0, 16 * (i - j), zero4());
            float* Ub = sU + w * 16 * LU;
#pragma unroll
            for (int r = 0; r < 4; ++r) Ub[(4 * lg + r) * LU + ln] = Uv[r];
            // T_ij = -T_ii U (same wavefront: its own LDS writes precede its reads)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the U tile is in LDS
            const f32x4 Tv = mm4(sT + 16 * i * LL + 16 * i, LL, 1, Ub, LU, 1, 0, 16, zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * lg + r) * LL + 16 * j + ln] = -Tv[r];
        }
        __syncthreads();
    }
    float* R = rec + ((size_t)slot * H + h) * RL::FLOATS;
    ST* const RW = rec_w<ST, KD>(R);
    ST* const RQ = rec_qt<ST, KD>(R);
    // W = T (beta Gamma K) on the wavefront's row tile (T is zero past column 16 w + 15)
#pragma unroll
    for (int jc = 0; jc < NJ; ++jc) {
        f32x4 Wv;
        if constexpr (B16)
            Wv = mmg(sT + 16 * w * LL, LL, 1, sK + 16 * jc, LK, 1, 0, 16 * (w + 1), zero4());
        else
            Wv = mmx<ST>(sT + 16 * w * LL, LL, 1, sK + 16 * jc, LK, 1, 0, 16 * (w + 1), zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sW[tr[r] * LK + 16 * jc + ln] = Elem<ST>::from_f(Wv[r]);
            RW[tr[r] * KD + 16 * jc + ln] = Elem<ST>::from_f(Wv[r]);
        }
    }
    __syncthreads();
    // Qt = scale Gamma Q - P W
#pragma unroll
    for (int jc = 0; jc < NJ; ++jc) {
        f32x4 PW;
        if constexpr (B16)
            PW = mmg(sP + 16 * w * LL, LL, 1, sW + 16 * jc, LK, 1, 0, 16 * (w + 1), zero4());
        else
            PW = mmx<ST>(sP + 16 * w * LL, LL, 1, sW + 16 * jc, LK, 1, 0, 16 * (w + 1), zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tr[r], c = 16 * jc + ln;
            RQ[t * KD + c] = Elem<ST>::from_f(scale * sGam[t] * Elem<ST>::to_f(sQ[t * LK + c]) - PW[r]);
        }
    }
    for (int i = tid; i < BC * BC; i += NT) {
        rec_t<ST, KD>(R)[i] = Elem<ST>::from_f(sT[(i / BC) * LL + i % BC]);
        // bf16 inputs: T^T follows T in the float32-sized region (the gradient kernel reads T by columns from it)
        if constexpr (sizeof(ST) == 2) rec_t<ST, KD>(R)[BC * BC + i] = Elem<ST>::from_f(sT[(i % BC) * LL + i / BC]);
    }
    if (tid < BC) {
        const float G = sG[tid], GL = sG[BC - 1];
        R[RL::C_OFF + tid] = G;
        R[RL::C_OFF + 64 + tid] = expf(G);
        R[RL::C_OFF + 128 + tid] = expf(GL - G);
        R[RL::C_OFF + 192 + tid] = sB[tid];
    }
}

// The prep for bf16 inputs, in 79 KB of LDS so that two workgroups share a CU: K and Q rows in bf16; the Q rows'
// block holds the U tiles of the off-diagonal solve once Q K^T is formed, then W; P in bf16 (it enters only P W);
// scale Gamma Q of the lane's own Q~ entries kept in registers from the start. The same steps as
// gdn_bwd_prep_kernel.
template <int KD>
__global__ __launch_bounds__(2 * NT) void gdn_bwd_prep16_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                            const float* __restrict__ g, const float* __restrict__ beta,
                                                            const int2* __restrict__ table, const int32_t* __restrict__ cu,
                                                            int T, int H, int nc, float scale, float* __restrict__ rec) {
    typedef BwdRec<KD> RL;
    typedef Elem<bf16_t> El;
    constexpr int NG = 2 * NT;  // eight wavefronts: (token tile w, half hv)
    constexpr int KP = KD + 8, CP = BC + 8, LL = BC + 1, LU = 17, NJ = KD / 16;
    constexpr int OFF_K = 0, OFF_QW = OFF_K + BC * KP * 2, OFF_A = OFF_QW + BC * KP * 2, OFF_T = OFF_A + BC * LL * 4,
                  OFF_P = OFF_T + BC * LL * 4, OFF_S = OFF_P + BC * CP * 2, BYTES = OFF_S + 3 * BC * 4;
    static_assert(4 * 16 * LU * 4 <= BC * KP * 2, "the U tiles fit the Q rows' block");
    static_assert(BYTES <= 80 * 1024, "two workgroups per CU");
    __shared__ __align__(16) uint8_t smem[BYTES];
    bf16_t* const sK = reinterpret_cast<bf16_t*>(smem + OFF_K);
    bf16_t* const sQ = reinterpret_cast<bf16_t*>(smem + OFF_QW);  // Q rows, then (float) U tiles, then W rows
    bf16_t* const sW = sQ;
    float* const sU = reinterpret_cast<float*>(smem + OFF_QW);
    float* const sA = reinterpret_cast<float*>(smem + OFF_A);
    float* const sT = reinterpret_cast<float*>(smem + OFF_T);
    bf16_t* const sP = reinterpret_cast<bf16_t*>(smem + OFF_P);
    float* const sG = reinterpret_cast<float*>(smem + OFF_S);
    float* const sB = sG + BC;
    float* const sGam = sB + BC;
    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const long row0 = (long)b * T + t0;
    {
        Tile<bf16_t, BC, KD, NG> tk, tq;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tq.load(q + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tk.template store_raw<KP>(sK);
        tq.template store_raw<KP>(sQ);
    }
    if (tid < BC) {
        const float gv = tid < L ? g[(row0 + tid) * H + h] : 0.f;
        sB[tid] = tid < L ? beta[(row0 + tid) * H + h] : 0.f;
        const float G = wave_inclusive_scan(gv);
        sG[tid] = G;
        sGam[tid] = expf(G);
    }
    __syncthreads();
    // wavefront wi: token tile w; half hv takes the column tiles j = 2 hv, 2 hv + 1 of A and P and the key tiles
    // HJ hv .. HJ hv + HJ - 1 of W and Qt
    const int wi = tid >> 6, w = wi & 3, hv = wi >> 2, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    constexpr int HJ = NJ / 2;
    int tr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) tr[r] = 16 * w + 4 * lg + r;
    // scale Gamma Q at the lane's Q~ entries (rows tr[r], columns 16 jc + ln)
    float qg[HJ][4];
#pragma unroll
    for (int jj = 0; jj < HJ; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) qg[jj][r] = scale * sGam[tr[r]] * bf2f(sQ[tr[r] * KP + 16 * (HJ * hv + jj) + ln]);
    // A = diag(beta) (D_strict o K K^T) and P = scale (D o Q K^T) on the wavefront's row tile
    for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * hv + jj;
        f32x4 kk = zero4(), qk = zero4();
        if (j <= w) {
            kk = mmb(sK + 16 * w * KP, KP, sK + 16 * j * KP, KP, 0, KD, kk);
            qk = mmb(sQ + 16 * w * KP, KP, sK + 16 * j * KP, KP, 0, KD, qk);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tr[r], s2 = 16 * j + ln;
            const float d = s2 <= t ? expf(sG[t] - sG[s2]) : 0.f;
            sA[t * LL + s2] = s2 < t ? sB[t] * d * kk[r] : 0.f;
            sP[t * CP + s2] = f2bf(scale * d * qk[r]);
            sT[t * LL + s2] = 0.f;
        }
    }
    __syncthreads();
    // diagonal blocks: wavefront w of half 0 inverts block w, lane j < 16 solving column j in registers
    if (hv == 0 && lane < 16) {
        const int o = 16 * w, j = lane;
        float xs[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = i == j ? 1.f : 0.f;
#pragma unroll
            for (int s2 = 0; s2 < i; ++s2) x -= sA[(o + i) * LL + o + s2] * xs[s2];
            xs[i] = x;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(o + i) * LL + o + j] = xs[i];
    }
    // (K scaled by beta Gamma per token, for W: K is not read again as itself)
    for (int i = tid; i < BC * KD; i += NG) {
        const int t = i / KD, c = i % KD;
        sK[t * KP + c] = f2bf(bf2f(sK[t * KP + c]) * (sB[t] * sGam[t]));
    }
    __syncthreads();
    // off-diagonal blocks, one block diagonal dd at a time: block (i, j = i - dd) by wavefront i of half 0
    for (int dd = 1; dd < 4; ++dd) {
        const int i = w, j = w - dd;
        if (hv == 0 && j >= 0) {
            const f32x4 Uv = mm4(sA + 16 * i * LL + 16 * j, LL, 1, sT + 16 * j * LL + 16 * j, LL, 1, 0, 16 * (i - j), zero4());
            float* Ub = sU + w * 16 * LU;
#pragma unroll
            for (int r = 0; r < 4; ++r) Ub[(4 * lg + r) * LU + ln] = Uv[r];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the U tile is in LDS
            const f32x4 Tv = mm4(sT + 16 * i * LL + 16 * i, LL, 1, Ub, LU, 1, 0, 16, zero4());
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[(16 * i + 4 * lg + r) * LL + 16 * j + ln] = -Tv[r];
        }
        __syncthreads();
    }
    float* R = rec + ((size_t)slot * H + h) * RL::FLOATS;
    bf16_t* const RW = rec_w<bf16_t, KD>(R);
    bf16_t* const RQ = rec_qt<bf16_t, KD>(R);
    // W = T (beta Gamma K) on the wavefront's row tile (T is zero past column 16 w + 15)
#pragma unroll
    for (int jj = 0; jj < HJ; ++jj) {
        const int jc = HJ * hv + jj;
        const f32x4 Wv = mmg(sT + 16 * w * LL, LL, 1, sK + 16 * jc, KP, 1, 0, 16 * (w + 1), zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sW[tr[r] * KP + 16 * jc + ln] = f2bf(Wv[r]);
            RW[tr[r] * KD + 16 * jc + ln] = f2bf(Wv[r]);
        }
    }
    __syncthreads();
    // Qt = scale Gamma Q - P W
#pragma unroll
    for (int jj = 0; jj < HJ; ++jj) {
        const int jc = HJ * hv + jj;
        const f32x4 PW = mmg(sP + 16 * w * CP, CP, 1, sW + 16 * jc, KP, 1, 0, 16 * (w + 1), zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) RQ[tr[r] * KD + 16 * jc + ln] = f2bf(qg[jj][r] - PW[r]);
    }
    for (int i = tid; i < BC * BC; i += NG) {
        rec_t<bf16_t, KD>(R)[i] = f2bf(sT[(i / BC) * LL + i % BC]);
        rec_t<bf16_t, KD>(R)[BC * BC + i] = f2bf(sT[(i % BC) * LL + i / BC]);  // T^T (read by columns)
    }
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
// chunk (float32 [slot][H][V][K]), on float32 MFMA tiles. Wavefront w holds key tiles JPW w .. JPW w + JPW - 1
// of the slice's state (lane: rows 4 lg + r, key 16 jc + ln) and forms token tile w of X and R.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_states_kernel(const ST* __restrict__ k, const ST* __restrict__ v,
                                                            const float* __restrict__ h0, const int32_t* __restrict__ cu,
                                                            const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                            int T, int H, int V, int n_seq, int nc, int nvs,
                                                            float* __restrict__ states) {
    typedef BwdRec<KD> RL;
    constexpr int LK = KD + 1, LL = BC + 1, LV = 17, JPW = KD / 64;
    __shared__ float sK[BC * LK], sS[16 * LK], sT[BC * LL], sV[BC * LV], sZ[BC * LV], sC[256];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    int b, bos, eos, slot0;
    seq_of(n, cu, chunk_off, T, nc, b, bos, eos, slot0);
    const int nch = (eos - bos + BC - 1) / BC;
    f32x4 S[JPW];
#pragma unroll
    for (int i = 0; i < JPW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[i][r] = h0 ? h0[(((size_t)n * H + h) * V + v0 + 4 * lg + r) * KD + 16 * (JPW * w + i) + ln] : 0.f;
    Tile<ST, BC, KD> tk;
    Tile<ST, BC, BC> tt;
    Tile<ST, BC, 16> tv;
    float cf = 0.f;
    auto issue = [&](int ci) __attribute__((always_inline)) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
        const float* R = rec + ((size_t)(slot0 + ci) * H + h) * RL::FLOATS;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tt.load(rec_t<ST, KD>(R), BC, BC);
        tv.load(v + (row0 * H + h) * (long)V + v0, (long)H * V, L);
        cf = R[RL::C_OFF + tid];
    };
    if (nch > 0) issue(0);
    for (int ci = 0; ci < nch; ++ci) {
        float* Sout = states + (((size_t)(slot0 + ci) * H + h) * V + v0) * KD;
#pragma unroll
        for (int i = 0; i < JPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * lg + r, c = 16 * (JPW * w + i) + ln;
                Sout[row * KD + c] = S[i][r];
                sS[row * LK + c] = S[i][r];
            }
        tk.store(sK);
        tt.store(sT);
        tv.store(sV);
        sC[tid] = cf;
        __syncthreads();
        if (ci + 1 < nch) issue(ci + 1);
        // Z = diag(beta) (V - diag(Gamma) K S^T) on token tile w
        const f32x4 X = mmx<ST>(sK + 16 * w * LK, LK, 1, sS, 1, LK, 0, KD, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * w + 4 * lg + r;
            sZ[t * LV + ln] = sC[192 + t] * (sV[t * LV + ln] - sC[64 + t] * X[r]);
        }
        __syncthreads();
        // e R = e T Z (into sV, no longer needed)
        const f32x4 Rv = mmx<ST>(sT + 16 * w * LL, LL, 1, sZ, LV, 1, 0, 16 * (w + 1), zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * w + 4 * lg + r;
            sV[t * LV + ln] = sC[128 + t] * Rv[r];
        }
        __syncthreads();
        // S <- Gamma_L S + (e R)^T K on the wavefront's key tiles
        const float gl = sC[64 + BC - 1];
#pragma unroll
        for (int i = 0; i < JPW; ++i) S[i] = mmx<ST>(sV, 1, LV, sK + 16 * (JPW * w + i), LK, 1, 0, BC, S[i] * gl);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------------------------
// Reverse chain: one 16-row slice of one (sequence, head), from dht (or zero) backwards, on float32 MFMA tiles.
// Before chunk c's step the slice holds the gradient of chunk c's exit state, stored as float32 [slot][H][V][K];
// after chunk 0 it is dh0. Wavefront w holds key tiles JPW w .. of the gradient and forms token tile w of Z.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_dstate_kernel(const ST* __restrict__ k, const ST* __restrict__ dout,
                                                            const float* __restrict__ dht, const int32_t* __restrict__ cu,
                                                            const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                            int T, int H, int V, int n_seq, int nc, int nvs,
                                                            float* __restrict__ dstates, float* __restrict__ dh0) {
    typedef BwdRec<KD> RL;
    constexpr int LK = KD + 1, LV = 17, LZ = BC + 1, JPW = KD / 64;
    __shared__ float sK[BC * LK], sW[BC * LK], sQt[BC * LK], sD[16 * LK], sO[BC * LV], sZ[16 * LZ], sC[256];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    int b, bos, eos, slot0;
    seq_of(n, cu, chunk_off, T, nc, b, bos, eos, slot0);
    const int nch = (eos - bos + BC - 1) / BC;
    f32x4 dS[JPW];
#pragma unroll
    for (int i = 0; i < JPW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dS[i][r] = dht ? dht[(((size_t)n * H + h) * V + v0 + 4 * lg + r) * KD + 16 * (JPW * w + i) + ln] : 0.f;
    // chunk ci's K rows, W, Qt, coefficients and dO slice, loaded one chunk ahead (chunks run backwards)
    Tile<ST, BC, KD> tk, tw, tq;
    Tile<ST, BC, 16> to;
    float cf = 0.f;
    auto issue = [&](int ci) __attribute__((always_inline)) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
        const float* R = rec + ((size_t)(slot0 + ci) * H + h) * RL::FLOATS;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tw.load(rec_w<ST, KD>(R), KD, BC);
        tq.load(rec_qt<ST, KD>(R), KD, BC);
        to.load(dout + (row0 * H + h) * (long)V + v0, (long)H * V, L);
        cf = R[RL::C_OFF + tid];
    };
    if (nch > 0) issue(nch - 1);
    for (int ci = nch - 1; ci >= 0; --ci) {
        float* Dout = dstates + (((size_t)(slot0 + ci) * H + h) * V + v0) * KD;
#pragma unroll
        for (int i = 0; i < JPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 4 * lg + r, c = 16 * (JPW * w + i) + ln;
                Dout[row * KD + c] = dS[i][r];
                sD[row * LK + c] = dS[i][r];
            }
        tk.store(sK);
        tw.store(sW);
        tq.store(sQt);
        to.store(sO);
        sC[tid] = cf;
        __syncthreads();
        if (ci > 0) issue(ci - 1);
        // Z[r][t] = e_t (dS' K^T)[r][t] on token tile w
        const f32x4 Zt = mmx<ST>(sD, LK, 1, sK + 16 * w * LK, 1, LK, 0, KD, zero4());
        const float et = sC[128 + 16 * w + ln];
#pragma unroll
        for (int r = 0; r < 4; ++r) sZ[(4 * lg + r) * LZ + 16 * w + ln] = et * Zt[r];
        __syncthreads();
        // dS = Gamma_L dS' + dO^T Qt - Z W on the wavefront's key tiles
        const float gl = sC[64 + BC - 1];
#pragma unroll
        for (int i = 0; i < JPW; ++i) {
            const int jc = JPW * w + i;
            const f32x4 a = mmx<ST>(sO, 1, LV, sQt + 16 * jc, LK, 1, 0, BC, dS[i] * gl);
            const f32x4 zw = mmx<ST>(sZ, LZ, 1, sW + 16 * jc, LK, 1, 0, BC, zero4());
            dS[i] = a - zw;
        }
        __syncthreads();
    }
    if (dh0) {
#pragma unroll
        for (int i = 0; i < JPW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dh0[(((size_t)n * H + h) * V + v0 + 4 * lg + r) * KD + 16 * (JPW * w + i) + ln] = dS[i][r];
    }
}

// ---------------------------------------------------------------------------------------------------------
// Gradients of one (chunk slot, head), on float32 MFMA tiles: wavefront w owns token rows 16 w .. 16 w + 15 of
// every product. The value dimension runs in 16-row slices (entry state, exit-state gradient and dO of the
// slice, the next slice's loading ahead); dP, dT, dq and dk accumulate over the slices in registers; then the
// solve's and the gate's terms. P (scale D o Q K^T) is kept rather than the raw Q K^T: the gate term
// scale dP D Q K^T is dP o P.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_grad_kernel(
    const ST* __restrict__ q, const ST* __restrict__ k, const ST* __restrict__ v, const ST* __restrict__ dout,
    const float* __restrict__ rec, const float* __restrict__ states, const float* __restrict__ dstates,
    const int2* __restrict__ table, const int32_t* __restrict__ cu, int T, int H, int V, int nc, float scale,
    ST* __restrict__ dq, ST* __restrict__ dk, ST* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta) {
    typedef BwdRec<KD> RL;
    constexpr int LK = KD + 1, LL = BC + 1, LV = 17, NJ = KD / 16;
    __shared__ float sK[BC * LK], sQ[BC * LK], sT[BC * LL], sP[BC * LL], sKK[BC * LL], sC[256];
    // per-slice region; after the slices it holds dT (then U, then F) and scale D o dP
    constexpr int SLICE_FLOATS = 2 * 16 * LK + 5 * BC * LV > 2 * BC * LL ? 2 * 16 * LK + 5 * BC * LV : 2 * BC * LL;
    __shared__ float sX[SLICE_FLOATS];
    float* const sS = sX;               // [16][LK] entry state of the slice
    float* const sD = sX + 16 * LK;     // [16][LK] exit-state gradient of the slice
    float* const sO = sX + 32 * LK;     // [64][LV] dO of the slice
    float* const sZ = sO + BC * LV;     // [64][LV] Z = diag(beta) Y
    float* const sR = sZ + BC * LV;     // [64][LV] R
    float* const sdR = sR + BC * LV;    // [64][LV] dR
    float* const sdX = sdR + BC * LV;   // [64][LV] dX
    float* const sdT = sX;              // [64][LL] after the slices: dT, then U = dT T^T, then F
    float* const sDP = sX + BC * LL;    // [64][LL] after the slices: scale D o dP
    __shared__ float sDG[BC], sEE[BC], sRed[NT / 64], sCol[NT];

    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const long row0 = (long)b * T + t0;
    const float* Rc = rec + ((size_t)slot * H + h) * RL::FLOATS;
    {
        Tile<ST, BC, KD> tk, tq;
        Tile<ST, BC, BC> tt;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tq.load(q + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tt.load(rec_t<ST, KD>(Rc), BC, BC);
        sC[tid] = Rc[RL::C_OFF + tid];
        tk.store(sK);
        tq.store(sQ);
        tt.store(sT);
    }
    __syncthreads();
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    // the lane's C-tile rows: tokens tr[r] = 16 w + 4 lg + r; its A-operand row: token 16 w + ln
    int tr[4];
    float Gr[4], gam[4], ee[4], bb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        tr[r] = 16 * w + 4 * lg + r;
        Gr[r] = sC[tr[r]];
        gam[r] = sC[64 + tr[r]];
        ee[r] = sC[128 + tr[r]];
        bb[r] = sC[192 + tr[r]];
    }
    const float gq_a = scale * sC[64 + 16 * w + ln], e_a = sC[128 + 16 * w + ln];
    const float gl = sC[64 + BC - 1];
    // P = scale (D o Q K^T) (s <= t) and the raw K K^T (s < t) on the wavefront's row tile
    for (int j = 0; j < 4; ++j) {
        f32x4 qk = zero4(), kk = zero4();
        if (j <= w) {
            qk = mmx<ST>(sQ + 16 * w * LK, LK, 1, sK + 16 * j * LK, 1, LK, 0, KD, qk);
            kk = mmx<ST>(sK + 16 * w * LK, LK, 1, sK + 16 * j * LK, 1, LK, 0, KD, kk);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tr[r], s2 = 16 * j + ln;
            sP[t * LL + s2] = s2 <= t ? scale * expf(Gr[r] - sC[s2]) * qk[r] : 0.f;
            sKK[t * LL + s2] = s2 < t ? kk[r] : 0.f;
        }
    }
    f32x4 aP[4], aT[4], aQ[NJ], aK[NJ];
#pragma unroll
    for (int j = 0; j < 4; ++j) aP[j] = aT[j] = zero4();
#pragma unroll
    for (int j = 0; j < NJ; ++j) aQ[j] = aK[j] = zero4();
    float pGam[4] = {0.f, 0.f, 0.f, 0.f}, pE[4] = {0.f, 0.f, 0.f, 0.f}, pB[4] = {0.f, 0.f, 0.f, 0.f}, pGL = 0.f;
    const int nvs = V / 16;
    Tile<float, 16, KD> ts, td;
    Tile<ST, BC, 16> to;
    auto issue = [&](int vs) __attribute__((always_inline)) {
        const int v0 = 16 * vs;
        ts.load(states + (((size_t)slot * H + h) * V + v0) * KD, KD, 16);
        td.load(dstates + (((size_t)slot * H + h) * V + v0) * KD, KD, 16);
        to.load(dout + (row0 * H + h) * (long)V + v0, (long)H * V, L);
    };
    issue(0);
    __syncthreads();
    for (int vs = 0; vs < nvs; ++vs) {
        const int v0 = 16 * vs;
        ts.store(sS);
        td.store(sD);
        to.store(sO);
        float vv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = tr[r] < L ? ld(v + ((row0 + tr[r]) * H + h) * (long)V + v0 + ln) : 0.f;
        if (vs + 1 < nvs) issue(vs + 1);
        __syncthreads();
        // X = K S^T, QS = Q S^T, KdS = K dS'^T on (token tile w, the slice's 16 values)
        const f32x4 X = mmx<ST>(sK + 16 * w * LK, LK, 1, sS, 1, LK, 0, KD, zero4());
        const f32x4 QS = mmx<ST>(sQ + 16 * w * LK, LK, 1, sS, 1, LK, 0, KD, zero4());
        const f32x4 KdS = mmx<ST>(sK + 16 * w * LK, LK, 1, sD, 1, LK, 0, KD, zero4());
        float Y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            Y[r] = vv[r] - gam[r] * X[r];
            sZ[tr[r] * LV + ln] = bb[r] * Y[r];
            pGam[r] += scale * sO[tr[r] * LV + ln] * QS[r];
        }
        __syncthreads();
        // R = T Z;  dR = P^T dO + e KdS
        const f32x4 R = mmx<ST>(sT + 16 * w * LL, LL, 1, sZ, LV, 1, 0, 16 * (w + 1), zero4());
        const f32x4 dRp = mmx<ST>(sP + 16 * w, 1, LL, sO, LV, 1, 16 * w, BC, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float dr = dRp[r] + ee[r] * KdS[r];
            sR[tr[r] * LV + ln] = R[r];
            sdR[tr[r] * LV + ln] = dr;
            pE[r] += R[r] * KdS[r];
        }
        __syncthreads();
        // dZ = T^T dR; dbeta, dY = dV, dX = -Gamma dY; dP += dO R^T, dT += dR Z^T
        const f32x4 dZ = mmx<ST>(sT + 16 * w, 1, LL, sdR, LV, 1, 16 * w, BC, zero4());
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pB[r] += Y[r] * dZ[r];
            const float dY = bb[r] * dZ[r];
            if (tr[r] < L) dv[((row0 + tr[r]) * H + h) * (long)V + v0 + ln] = Elem<ST>::from_f(dY);
            sdX[tr[r] * LV + ln] = -gam[r] * dY;
            pGam[r] -= dY * X[r];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            aP[j] = mmx<ST>(sO + 16 * w * LV, LV, 1, sR + 16 * j * LV, 1, LV, 0, 16, aP[j]);
            aT[j] = mmx<ST>(sdR + 16 * w * LV, LV, 1, sZ + 16 * j * LV, 1, LV, 0, 16, aT[j]);
        }
        for (int i = tid; i < 16 * KD; i += NT) pGL += sS[(i / KD) * LK + i % KD] * sD[(i / KD) * LK + i % KD];
        __syncthreads();
        // dq += scale Gamma dO S;  dk += dX S + e R dS'
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            aQ[j] = mmx<ST>(sO + 16 * w * LV, LV, 1, sS + 16 * j, LK, 1, 0, 16, aQ[j], gq_a);
            aK[j] = mmx<ST>(sdX + 16 * w * LV, LV, 1, sS + 16 * j, LK, 1, 0, 16, aK[j]);
            aK[j] = mmx<ST>(sR + 16 * w * LV, LV, 1, sD + 16 * j, LK, 1, 0, 16, aK[j], e_a);
        }
        __syncthreads();
    }
    // dT to LDS, U = dT T^T (T[s][j] is zero past j = s)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sdT[tr[r] * LL + 16 * j + ln] = aT[j][r];
    __syncthreads();
    f32x4 U[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) U[j] = mmx<ST>(sdT + 16 * w * LL, LL, 1, sT + 16 * j * LL, 1, LL, 0, 16 * (j + 1), zero4());
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) sdT[tr[r] * LL + 16 * j + ln] = U[j][r];
    __syncthreads();
    // dA = -T^T U on s < t (T[j][t] is zero below j = t); then the gate terms, F and scale D o dP
    float rowc[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 Fv[4], DPv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f32x4 dA = zero4();
        if (j <= w) dA = mmx<ST>(sT + 16 * w, 1, LL, sdT + 16 * j, LL, 1, 16 * w, BC, dA);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tr[r], s2 = 16 * j + ln;
            const float d = s2 <= t ? expf(Gr[r] - sC[s2]) : 0.f;
            const float a = s2 < t ? -dA[r] : 0.f;
            const float kk = sKK[t * LL + s2];
            pB[r] += a * d * kk;
            Fv[j][r] = a * bb[r] * d;
            DPv[j][r] = s2 <= t ? scale * d * aP[j][r] : 0.f;
            const float c = (s2 <= t ? aP[j][r] * sP[t * LL + s2] : 0.f) + Fv[j][r] * kk;
            rowc[r] += c;
            sKK[t * LL + s2] = c;  // own entry: K K^T is not read again
        }
    }
    __syncthreads();  // U is no longer read
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sdT[tr[r] * LL + 16 * j + ln] = Fv[j][r];
            sDP[tr[r] * LL + 16 * j + ln] = DPv[j][r];
        }
    __syncthreads();
    // dq += (scale D o dP) K;  dk += (scale D o dP)^T Q + F K + F^T K
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        aQ[j] = mmx<ST>(sDP + 16 * w * LL, LL, 1, sK + 16 * j, LK, 1, 0, 16 * (w + 1), aQ[j]);
        aK[j] = mmx<ST>(sDP + 16 * w, 1, LL, sQ + 16 * j, LK, 1, 16 * w, BC, aK[j]);
        aK[j] = mmx<ST>(sdT + 16 * w * LL, LL, 1, sK + 16 * j, LK, 1, 0, 16 * (w + 1), aK[j]);
        aK[j] = mmx<ST>(sdT + 16 * w, 1, LL, sK + 16 * j, LK, 1, 16 * w, BC, aK[j]);
    }
    // row sums over the 16 lanes of each row group; <dS', S> over the workgroup
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pGam[r] += __shfl_xor(pGam[r], o, 64);
            pE[r] += __shfl_xor(pE[r], o, 64);
            pB[r] += __shfl_xor(pB[r], o, 64);
            rowc[r] += __shfl_xor(rowc[r], o, 64);
        }
    for (int o = 1; o < 64; o <<= 1) pGL += __shfl_xor(pGL, o, 64);
    if (lane == 0) sRed[w] = pGL;
    if (ln == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sDG[tr[r]] = pGam[r] * gam[r] - pE[r] * ee[r] + rowc[r];
            sEE[tr[r]] = pE[r] * ee[r];
            if (tr[r] < L) dbeta[(row0 + tr[r]) * H + h] = pB[r];
        }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (tr[r] < L) {
                const long o = ((row0 + tr[r]) * H + h) * (long)KD + 16 * j + ln;
                dq[o] = Elem<ST>::from_f(aQ[j][r]);
                dk[o] = Elem<ST>::from_f(aK[j][r]);
            }
    __syncthreads();
    {
        // column sums of the gate terms: wavefront w over rows 16 w .. 16 w + 15, lane = column
        float part = 0.f;
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) part += sKK[(16 * w + tt) * LL + lane];
        sCol[tid] = part;
    }
    __syncthreads();
    if (tid < BC) {
        const float col = (sCol[tid] + sCol[64 + tid]) + (sCol[128 + tid] + sCol[192 + tid]);
        float dG = sDG[tid] - col;
        // G_L (token 63: padded tokens repeat the last real G) also carries e's and Gamma_L's terms
        float se = sEE[tid];
        for (int o = 1; o < 64; o <<= 1) se += __shfl_xor(se, o, 64);
        if (tid == BC - 1) {
            float gsum = 0.f;
#pragma unroll
            for (int ww = 0; ww < NT / 64; ++ww) gsum += sRed[ww];
            dG += se + gsum * gl;
        }
        // dg = the reverse cumulative sum of dG over the chunk: lane l scans dG of token 63 - l
        const float rev = __shfl(dG, BC - 1 - tid, 64);
        const float cs = wave_inclusive_scan(rev);
        const float dgt = __shfl(cs, BC - 1 - tid, 64);
        if (tid < L) dg[(row0 + tid) * H + h] = dgt;
    }
}

// ---------------------------------------------------------------------------------------------------------
// The gradient kernel for bf16 inputs, per (chunk slot, head): the products of gdn_bwd_grad_kernel on bf16 LDS
// operands. K, Q, T, T^T (from the record), P and the slices' state rows are kept in bf16, so every operand reaches
// its product by a 16-byte read of eight consecutive reduction elements (row form: A rows and B^T rows, k
// contiguous) or by two transposing reads (ds_read_b64_tr_b16) of a row-major block, which give a lane four
// consecutive rows of one column, the C-tile shape (column form: both operands indexed [k][m] and [k][n]). The
// value dimension goes in slices of 32, so the per-slice products (dP, dT, dq, dk) reduce 32 values per
// 16x16x32 MFMA. The products after the slices take their float operands as before and the bf16 ones from
// these arrays (mmg, the same bits as mm32).
// ---------------------------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint8_t lds8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

// column form: lane (ln, lg) gets M[r0 + 4 lg + i][c0 + ln], i = 0..3, of the row-major bf16 block M (pitch P
// elements, a multiple of 4; c0 a multiple of 4)
__device__ __forceinline__ i16x4 col4(const bf16_t* M, int P, int r0, int c0) {
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    const bf16_t* a = M + (r0 + 4 * lg + (ln >> 2)) * P + c0 + 4 * (ln & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(lds8*)a);
}
// the 32-deep column-form operand: rows r0 + 4 lg + i, then r0 + 16 + 4 lg + i
__device__ __forceinline__ bf16x8 col8(const bf16_t* M, int P, int r0, int c0) {
    return cat8(col4(M, P, r0, c0), col4(M, P, r0 + 16, c0));
}
// row form: lane (ln, lg) gets M[r0 + ln][k0 + 8 lg .. + 7] (pitch P a multiple of 8, k0 of 8)
__device__ __forceinline__ bf16x8 row8(const bf16_t* M, int P, int r0, int k0) {
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    return *(const lds_bf16x8_t*)(lds8*)(M + (r0 + ln) * P + k0 + 8 * lg);
}
// C tile (rows r0 + 4 lg + i, column c0 + ln) into a row-major bf16 block, and transposed (row c0 + ln, columns
// r0 + 4 lg .. + 3: one 8-byte write)
__device__ __forceinline__ void put_rows(bf16_t* M, int P, int r0, int c0, f32x4 c) {
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) M[(r0 + 4 * lg + i) * P + c0 + ln] = f2bf(c[i]);
}
__device__ __forceinline__ void put_cols(bf16_t* M, int P, int r0, int c0, f32x4 c) {
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    *(lds_i16x4_t*)(lds8*)(M + (c0 + ln) * P + r0 + 4 * lg) = Elem<bf16_t>::pack(c);
}

template <int KD>
__global__ __launch_bounds__(2 * NT) void gdn_bwd_grad16_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ rec, const float* __restrict__ states,
    const float* __restrict__ dstates, const int2* __restrict__ table, const int32_t* __restrict__ cu, int T, int H,
    int V, int nc, float scale, bf16_t* __restrict__ dq, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta) {
    typedef BwdRec<KD> RL;
    typedef Elem<bf16_t> El;
    constexpr int NG = 2 * NT;   // eight wavefronts: two per token tile
    constexpr int KP = KD + 8;   // bf16 pitch of K, Q and the state rows
    constexpr int CP = BC + 8;   // bf16 pitch of 64-wide rows (T, T^T, P, and the slices' transposed blocks)
    constexpr int SW = 32;       // values per slice
    constexpr int VP = SW + 8;   // bf16 pitch of a slice's token rows
    constexpr int LL = BC + 1;   // float pitch of P, K K^T, D o dP terms
    constexpr int NJ = KD / 16, HJ = NJ / 2;
    __shared__ __align__(16) bf16_t sK[BC * KP], sQ[BC * KP], sT[BC * CP], sTt[BC * CP], sPb[BC * CP];
    __shared__ float sP[BC * LL], sKK[BC * LL], sC[256];
    // per-slice region (bf16); after the slices it holds dT (then U, then F), F^T and scale D o dP both ways
    constexpr int SLICE_BYTES = (2 * SW * KP + 5 * BC * VP + 3 * SW * CP) * 2, POST_BYTES = 4 * BC * CP * 2;
    __shared__ __align__(16) uint8_t sX[SLICE_BYTES > POST_BYTES ? SLICE_BYTES : POST_BYTES];
    bf16_t* const sS = reinterpret_cast<bf16_t*>(sX);  // [SW][KP] entry state rows of the slice
    bf16_t* const sD = sS + SW * KP;                    // [SW][KP] exit-state gradient rows
    bf16_t* const sO = sD + SW * KP;                    // [BC][VP] dO
    bf16_t* const sV = sO + BC * VP;                    // [BC][VP] V
    bf16_t* const sZ = sV + BC * VP;                    // [BC][VP] Z = diag(beta) Y
    bf16_t* const sR = sZ + BC * VP;                    // [BC][VP] R
    bf16_t* const sdR = sR + BC * VP;                   // [BC][VP] dR
    bf16_t* const sOt = sdR + BC * VP;                  // [SW][CP] dO^T
    bf16_t* const sRt = sOt + SW * CP;                  // [SW][CP] R^T
    bf16_t* const sXt = sRt + SW * CP;                  // [SW][CP] dX^T
    // per-token partial sums of the two wavefronts of a token tile; the workgroup's column sums and <dS', S>
    __shared__ float sDG[2][BC], sEE[2][BC], sDB[2][BC], sRed[NG / 64], sCol[NG];

    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const long row0 = (long)b * T + t0;
    const float* Rc = rec + ((size_t)slot * H + h) * RL::FLOATS;
    {
        Tile<bf16_t, BC, KD, NG> tk, tq;
        Tile<bf16_t, BC, BC, NG> tt, ttt;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tq.load(q + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tt.load(rec_t<bf16_t, KD>(Rc), BC, BC);
        ttt.load(rec_t<bf16_t, KD>(Rc) + BC * BC, BC, BC);
        if (tid < 256) sC[tid] = Rc[RL::C_OFF + tid];
        tk.template store_raw<KP>(sK);
        tq.template store_raw<KP>(sQ);
        tt.template store_raw<CP>(sT);
        ttt.template store_raw<CP>(sTt);
    }
    __syncthreads();
    // wavefront wi: token tile w and half hv (the slice's value tile hv, the key tiles HJ hv .. HJ hv + HJ - 1,
    // the token column tiles 2 hv, 2 hv + 1); a light and a heavy token tile share each SIMD
    const int wi = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int w = wi < 4 ? (wi & 1) : 3 - (wi & 1), hv = (wi >> 1) & 1;
    // the lane's C-tile rows: tokens tr[r] = 16 w + 4 lg + r
    int tr[4];
    float Gr[4], gam[4], ee[4], bb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        tr[r] = 16 * w + 4 * lg + r;
        Gr[r] = sC[tr[r]];
        gam[r] = sC[64 + tr[r]];
        ee[r] = sC[128 + tr[r]];
        bb[r] = sC[192 + tr[r]];
    }
    const float gl = sC[64 + BC - 1];
    // P = scale (D o Q K^T) (s <= t) and the raw K K^T (s < t) on the wavefront's two tiles
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * hv + jj;
        f32x4 qk = zero4(), kk = zero4();
        if (j <= w) {
            qk = mmb(sQ + 16 * w * KP, KP, sK + 16 * j * KP, KP, 0, KD, qk);
            kk = mmb(sK + 16 * w * KP, KP, sK + 16 * j * KP, KP, 0, KD, kk);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tr[r], s2 = 16 * j + ln;
            const float pv = s2 <= t ? scale * expf(Gr[r] - sC[s2]) * qk[r] : 0.f;
            sP[t * LL + s2] = pv;
            sPb[t * CP + s2] = f2bf(pv);
            sKK[t * LL + s2] = s2 < t ? kk[r] : 0.f;
        }
    }
    f32x4 aP[2], aT[2], aQ[HJ], aK[HJ], aK2[HJ];
#pragma unroll
    for (int j = 0; j < 2; ++j) aP[j] = aT[j] = zero4();
#pragma unroll
    for (int j = 0; j < HJ; ++j) aQ[j] = aK[j] = aK2[j] = zero4();
    float pGam[4] = {0.f, 0.f, 0.f, 0.f}, pE[4] = {0.f, 0.f, 0.f, 0.f}, pB[4] = {0.f, 0.f, 0.f, 0.f}, pGL = 0.f;
    const int nvs = V / SW;
    Tile<float, SW, KD, NG> ts, td;
    Tile<bf16_t, BC, SW, NG> to, tv;
    auto issue = [&](int vs) __attribute__((always_inline)) {
        const int v0 = SW * vs;
        ts.load(states + (((size_t)slot * H + h) * V + v0) * KD, KD, SW);
        td.load(dstates + (((size_t)slot * H + h) * V + v0) * KD, KD, SW);
        to.load(dout + (row0 * H + h) * (long)V + v0, (long)H * V, L);
        tv.load(v + (row0 * H + h) * (long)V + v0, (long)H * V, L);
    };
    issue(0);
    __syncthreads();
    const int vt = hv;  // the wavefront's value tile of the slice
    for (int vs = 0; vs < nvs; ++vs) {
        const int v0 = SW * vs;
        // the slice's operands to LDS: state rows in bf16 (<S, dS'> in float32 from the same registers), dO and V
        // rows, dO^T
#pragma unroll
        for (int p = 0; p < decltype(ts)::PER; ++p) {
            const int idx = tid + NG * p, row = idx / decltype(ts)::PPR, col = (idx % decltype(ts)::PPR) * 4;
            if (idx < decltype(ts)::PIECES) {
                const f32x4 sv = __builtin_bit_cast(f32x4, ts.r[p]), dv4 = __builtin_bit_cast(f32x4, td.r[p]);
                pGL += (sv[0] * dv4[0] + sv[1] * dv4[1]) + (sv[2] * dv4[2] + sv[3] * dv4[3]);
                *(lds_i16x4_t*)(lds8*)(sS + row * KP + col) = El::pack(sv);
                *(lds_i16x4_t*)(lds8*)(sD + row * KP + col) = El::pack(dv4);
            }
        }
        to.template store_raw<VP>(sO);
        tv.template store_raw<VP>(sV);
#pragma unroll
        for (int p = 0; p < decltype(to)::PER; ++p) {
            const int idx = tid + NG * p, row = idx / decltype(to)::PPR, col = (idx % decltype(to)::PPR) * 8;
            if (idx < decltype(to)::PIECES)
#pragma unroll
                for (int e = 0; e < 8; ++e) sOt[(col + e) * CP + row] = unit_of<bf16_t>(to.r[p], e);
        }
        if (vs + 1 < nvs) issue(vs + 1);
        __syncthreads();
        // X = K S^T, QS = Q S^T, KdS = K dS'^T on (token tile w, value tile vt): row form
        const f32x4 X = mmb(sK + 16 * w * KP, KP, sS + 16 * vt * KP, KP, 0, KD, zero4());
        const f32x4 QS = mmb(sQ + 16 * w * KP, KP, sS + 16 * vt * KP, KP, 0, KD, zero4());
        const f32x4 KdS = mmb(sK + 16 * w * KP, KP, sD + 16 * vt * KP, KP, 0, KD, zero4());
        f32x4 Y;
        {
            const f32x4 vv = El::unpack(col4(sV, VP, 16 * w, 16 * vt)), oo = El::unpack(col4(sO, VP, 16 * w, 16 * vt));
            f32x4 z;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Y[r] = vv[r] - gam[r] * X[r];
                z[r] = bb[r] * Y[r];
                pGam[r] += scale * oo[r] * QS[r];
            }
            put_rows(sZ, VP, 16 * w, 16 * vt, z);
        }
        __syncthreads();
        // R = T Z (column form: T^T rows give T by columns); dR = P^T dO + e KdS (column form, P rows)
        {
            f32x4 R = zero4(), dRp = zero4(), dR;
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32) {
                if (k0 < 16 * (w + 1)) R = mma32(col8(sTt, CP, k0, 16 * w), col8(sZ, VP, k0, 16 * vt), R);
                if (k0 + 32 > 16 * w) dRp = mma32(col8(sPb, CP, k0, 16 * w), col8(sO, VP, k0, 16 * vt), dRp);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                dR[r] = dRp[r] + ee[r] * KdS[r];
                pE[r] += R[r] * KdS[r];
            }
            put_rows(sR, VP, 16 * w, 16 * vt, R);
            put_cols(sRt, CP, 16 * w, 16 * vt, R);
            put_rows(sdR, VP, 16 * w, 16 * vt, dR);
        }
        __syncthreads();
        // dZ = T^T dR (column form, T rows); dbeta, dY = dV, dX = -Gamma dY
        {
            f32x4 dZ = zero4(), dX;
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 + 32 > 16 * w) dZ = mma32(col8(sT, CP, k0, 16 * w), col8(sdR, VP, k0, 16 * vt), dZ);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pB[r] += Y[r] * dZ[r];
                const float dY = bb[r] * dZ[r];
                if (tr[r] < L) dv[((row0 + tr[r]) * H + h) * (long)V + v0 + 16 * vt + ln] = f2bf(dY);
                dX[r] = -gam[r] * dY;
                pGam[r] -= dY * X[r];
            }
            put_cols(sXt, CP, 16 * w, 16 * vt, dX);
        }
        // dP += dO R^T, dT += dR Z^T (row form over the slice's 32 values)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * hv + jj;
            aP[jj] = mmb(sO + 16 * w * VP, VP, sR + 16 * j * VP, VP, 0, SW, aP[jj]);
            aT[jj] = mmb(sdR + 16 * w * VP, VP, sZ + 16 * j * VP, VP, 0, SW, aT[jj]);
        }
        // dq += dO S, dk2 += R dS' (column form: dO^T, R^T by rows, S and dS' rows)
#pragma unroll
        for (int jj = 0; jj < HJ; ++jj) {
            const int j = HJ * hv + jj;
            aQ[jj] = mma32(col8(sOt, CP, 0, 16 * w), col8(sS, KP, 0, 16 * j), aQ[jj]);
            aK2[jj] = mma32(col8(sRt, CP, 0, 16 * w), col8(sD, KP, 0, 16 * j), aK2[jj]);
        }
        __syncthreads();  // both value tiles of dX^T are in LDS
        // dk += dX S
#pragma unroll
        for (int jj = 0; jj < HJ; ++jj) {
            const int j = HJ * hv + jj;
            aK[jj] = mma32(col8(sXt, CP, 0, 16 * w), col8(sS, KP, 0, 16 * j), aK[jj]);
        }
        __syncthreads();
    }
    // dq = scale Gamma (dO S), dk = dX S + e (R dS')
#pragma unroll
    for (int j = 0; j < HJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            aQ[j][r] *= scale * gam[r];
            aK[j][r] += ee[r] * aK2[j][r];
        }
    // after the slices, bf16 blocks in the slice region: dT, then U, then F by rows; F^T; scale D o dP by rows
    // and transposed
    bf16_t* const bF = reinterpret_cast<bf16_t*>(sX);  // [64][CP]
    bf16_t* const bFt = bF + BC * CP;
    bf16_t* const bD = bFt + BC * CP;
    bf16_t* const bDt = bD + BC * CP;
    static_assert(4 * BC * CP * 2 <= sizeof(sX), "post-slice blocks fit the slice region");
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) put_rows(bF, CP, 16 * w, 16 * (2 * hv + jj), aT[jj]);
    __syncthreads();
    // U = dT T^T (row form; T[s][j] is zero past j = s)
    f32x4 U[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * hv + jj;
        U[jj] = mmb(bF + 16 * w * CP, CP, sT + 16 * j * CP, CP, 0, 16 * (j + 1), zero4());
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) put_rows(bF, CP, 16 * w, 16 * (2 * hv + jj), U[jj]);
    __syncthreads();
    // dA = -T^T U on s < t (column form over the rows of T and U; T[k][t] is zero for k < t); then the gate
    // terms, F and scale D o dP
    float rowc[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 Fv[2], DPv[2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * hv + jj;
        f32x4 dA = zero4();
        if (j <= w) {
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 + 32 > 16 * w) dA = mma32(col8(sT, CP, k0, 16 * w), col8(bF, CP, k0, 16 * j), dA);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tr[r], s2 = 16 * j + ln;
            const float d = s2 <= t ? expf(Gr[r] - sC[s2]) : 0.f;
            const float a = s2 < t ? -dA[r] : 0.f;
            const float kk = sKK[t * LL + s2];
            pB[r] += a * d * kk;
            Fv[jj][r] = a * bb[r] * d;
            DPv[jj][r] = s2 <= t ? scale * d * aP[jj][r] : 0.f;
            const float c = (s2 <= t ? aP[jj][r] * sP[t * LL + s2] : 0.f) + Fv[jj][r] * kk;
            rowc[r] += c;
            sKK[t * LL + s2] = c;  // own entry: K K^T is not read again
        }
    }
    __syncthreads();  // U is no longer read
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * hv + jj;
        put_rows(bF, CP, 16 * w, 16 * j, Fv[jj]);
        put_cols(bFt, CP, 16 * w, 16 * j, Fv[jj]);
        put_rows(bD, CP, 16 * w, 16 * j, DPv[jj]);
        put_cols(bDt, CP, 16 * w, 16 * j, DPv[jj]);
    }
    __syncthreads();
    // dq += (scale D o dP) K;  dk += (scale D o dP)^T Q + F K + F^T K (column form over the tokens)
#pragma unroll
    for (int jj = 0; jj < HJ; ++jj) {
        const int j = HJ * hv + jj;
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 32) {
            const bf16x8 kcol = col8(sK, KP, k0, 16 * j);
            if (k0 < 16 * (w + 1)) {
                aQ[jj] = mma32(col8(bDt, CP, k0, 16 * w), kcol, aQ[jj]);
                aK[jj] = mma32(col8(bFt, CP, k0, 16 * w), kcol, aK[jj]);
            }
            if (k0 + 32 > 16 * w) {
                aK[jj] = mma32(col8(bD, CP, k0, 16 * w), col8(sQ, KP, k0, 16 * j), aK[jj]);
                aK[jj] = mma32(col8(bF, CP, k0, 16 * w), kcol, aK[jj]);
            }
        }
    }
    // row sums over the 16 lanes of each row group (each wavefront's share of the token's terms); <dS', S> over
    // the workgroup
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pGam[r] += __shfl_xor(pGam[r], o, 64);
            pE[r] += __shfl_xor(pE[r], o, 64);
            pB[r] += __shfl_xor(pB[r], o, 64);
            rowc[r] += __shfl_xor(rowc[r], o, 64);
        }
    for (int o = 1; o < 64; o <<= 1) pGL += __shfl_xor(pGL, o, 64);
    if (lane == 0) sRed[wi] = pGL;
    if (ln == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sDG[hv][tr[r]] = pGam[r] * gam[r] - pE[r] * ee[r] + rowc[r];
            sEE[hv][tr[r]] = pE[r] * ee[r];
            sDB[hv][tr[r]] = pB[r];
        }
#pragma unroll
    for (int jj = 0; jj < HJ; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (tr[r] < L) {
                const long o = ((row0 + tr[r]) * H + h) * (long)KD + 16 * (HJ * hv + jj) + ln;
                dq[o] = f2bf(aQ[jj][r]);
                dk[o] = f2bf(aK[jj][r]);
            }
    __syncthreads();
    {
        // column sums of the gate terms: wavefront wi over rows 8 wi .. 8 wi + 7, lane = column
        float part = 0.f;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) part += sKK[(8 * wi + tt) * LL + lane];
        sCol[tid] = part;
    }
    __syncthreads();
    if (tid < BC) {
        float col = 0.f;
#pragma unroll
        for (int ww = 0; ww < NG / 64; ++ww) col += sCol[64 * ww + tid];
        float dG = (sDG[0][tid] + sDG[1][tid]) - col;
        if (tid < L) dbeta[(row0 + tid) * H + h] = sDB[0][tid] + sDB[1][tid];
        // G_L (token 63: padded tokens repeat the last real G) also carries e's and Gamma_L's terms
        float se = sEE[0][tid] + sEE[1][tid];
        for (int o = 1; o < 64; o <<= 1) se += __shfl_xor(se, o, 64);
        if (tid == BC - 1) {
            float gsum = 0.f;
#pragma unroll
            for (int ww = 0; ww < NG / 64; ++ww) gsum += sRed[ww];
            dG += se + gsum * gl;
        }
        // dg = the reverse cumulative sum of dG over the chunk: lane l scans dG of token 63 - l
        const float rev = __shfl(dG, BC - 1 - tid, 64);
        const float cs = wave_inclusive_scan(rev);
        const float dgt = __shfl(cs, BC - 1 - tid, 64);
        if (tid < L) dg[(row0 + tid) * H + h] = dgt;
    }
}

// ---------------------------------------------------------------------------------------------------------
// The two chains for bf16 inputs, on the operand forms of gdn_bwd_grad16_kernel (bf16 LDS rows; row-form and
// column-form products): the same steps as gdn_bwd_states_kernel and gdn_bwd_dstate_kernel.
// ---------------------------------------------------------------------------------------------------------
template <int KD>
__global__ __launch_bounds__(NT) void gdn_bwd_states16_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                              const float* __restrict__ h0, const int32_t* __restrict__ cu,
                                                              const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                              int T, int H, int V, int n_seq, int nc, int nvs,
                                                              float* __restrict__ states) {
    typedef BwdRec<KD> RL;
    typedef Elem<bf16_t> El;
    constexpr int KP = KD + 8, CP = BC + 8, VP = 16 + 8, JPW = KD / 64;
    __shared__ __align__(16) bf16_t sK[BC * KP], sS[16 * KP], sTt[BC * CP], sV[BC * VP], sZ[BC * VP], sE[BC * VP];
    __shared__ float sC[256];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
    const int w = tid >> 6, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    int b, bos, eos, slot0;
    seq_of(n, cu, chunk_off, T, nc, b, bos, eos, slot0);
    const int nch = (eos - bos + BC - 1) / BC;
    f32x4 S[JPW];
#pragma unroll
    for (int i = 0; i < JPW; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[i][r] = h0 ? h0[(((size_t)n * H + h) * V + v0 + 4 * lg + r) * KD + 16 * (JPW * w + i) + ln] : 0.f;
    // the operands of a chunk in registers (three sets: chunk c's load is issued three steps before its step,
    // and the loop takes three steps per pass so that each set has fixed registers)
    struct Ops16 {
        Tile<bf16_t, BC, KD> tk;
        Tile<bf16_t, BC, BC> tt;
        Tile<bf16_t, BC, 16> tv;
        float cf;
    } opA, opB, opC;
    auto issue = [&](int ci, Ops16& o) __attribute__((always_inline)) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
        const float* R = rec + ((size_t)(slot0 + ci) * H + h) * RL::FLOATS;
        o.tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        o.tt.load(rec_t<bf16_t, KD>(R) + BC * BC, BC, BC);  // T^T
        o.tv.load(v + (row0 * H + h) * (long)V + v0, (long)H * V, L);
        o.cf = R[RL::C_OFF + tid];
    };
    auto step = [&](int ci, Ops16& o) __attribute__((always_inline)) {
        float* Sout = states + (((size_t)(slot0 + ci) * H + h) * V + v0) * KD;
#pragma unroll
        for (int i = 0; i < JPW; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r) Sout[(4 * lg + r) * KD + 16 * (JPW * w + i) + ln] = S[i][r];
            put_rows(sS, KP, 0, 16 * (JPW * w + i), S[i]);
        }
        o.tk.template store_raw<KP>(sK);
        o.tt.template store_raw<CP>(sTt);
        o.tv.template store_raw<VP>(sV);
        sC[tid] = o.cf;
        __syncthreads();
        if (ci + 3 < nch) issue(ci + 3, o);
        // Z = diag(beta) (V - diag(Gamma) K S^T) on token tile w (row form)
        const f32x4 X = mmb(sK + 16 * w * KP, KP, sS, KP, 0, KD, zero4());
        const f32x4 vv = El::unpack(col4(sV, VP, 16 * w, 0));
        f32x4 z;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * w + 4 * lg + r;
            z[r] = sC[192 + t] * (vv[r] - sC[64 + t] * X[r]);
        }
        put_rows(sZ, VP, 16 * w, 0, z);
        __syncthreads();
        // e R = e T Z (column form, T^T rows)
        f32x4 Rv = zero4();
#pragma unroll
        for (int k0 = 0; k0 < BC; k0 += 32)
            if (k0 < 16 * (w + 1)) Rv = mma32(col8(sTt, CP, k0, 16 * w), col8(sZ, VP, k0, 0), Rv);
#pragma unroll
        for (int r = 0; r < 4; ++r) Rv[r] *= sC[128 + 16 * w + 4 * lg + r];
        put_rows(sE, VP, 16 * w, 0, Rv);
        __syncthreads();
        // S <- Gamma_L S + (e R)^T K on the wavefront's key tiles (column form)
        const float gl = sC[64 + BC - 1];
#pragma unroll
        for (int i = 0; i < JPW; ++i) {
            f32x4 acc = S[i] * gl;
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32) acc = mma32(col8(sE, VP, k0, 0), col8(sK, KP, k0, 16 * (JPW * w + i)), acc);
            S[i] = acc;
        }
        __syncthreads();
    };
    if (nch > 0) issue(0, opA);
    if (nch > 1) issue(1, opB);
    if (nch > 2) issue(2, opC);
    for (int ci = 0; ci < nch; ci += 3) {
        step(ci, opA);
        if (ci + 1 < nch) step(ci + 1, opB);
        if (ci + 2 < nch) step(ci + 2, opC);
    }
}

template <int KD>
__global__ __launch_bounds__(2 * NT) void gdn_bwd_dstate16_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ dout,
                                                                  const float* __restrict__ dht, const int32_t* __restrict__ cu,
                                                                  const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                                  int T, int H, int V, int n_seq, int nc, int nvs,
                                                                  float* __restrict__ dstates, float* __restrict__ dh0) {
    typedef BwdRec<KD> RL;
    constexpr int NG = 2 * NT;  // eight wavefronts: (token tile w, half hv)
    constexpr int KP = KD + 8, VP = 16 + 8, JPW = KD / 64;
    __shared__ __align__(16) bf16_t sK[BC * KP], sW[BC * KP], sQt[BC * KP], sD[16 * KP], sO[BC * VP], sZt[BC * VP];
    __shared__ float sC[256];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
    // wavefront wi: token tile w for Z (half 0), key tile JPW w + hv of the state gradient (for K = 64 the
    // wavefronts of half 1 hold none)
    const int wi = tid >> 6, w = wi & 3, hv = wi >> 2, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const bool own = hv < JPW;
    const int jc = JPW * w + hv;
    int b, bos, eos, slot0;
    seq_of(n, cu, chunk_off, T, nc, b, bos, eos, slot0);
    const int nch = (eos - bos + BC - 1) / BC;
    f32x4 dS = zero4();
    if (own && dht)
#pragma unroll
        for (int r = 0; r < 4; ++r) dS[r] = dht[(((size_t)n * H + h) * V + v0 + 4 * lg + r) * KD + 16 * jc + ln];
    // chunk ci's K rows, W, Qt, coefficients and dO slice in registers (three sets: a chunk's load is issued
    // three steps before its step, chunks running backwards, and the loop takes three steps per pass so that
    // each set has fixed registers)
    struct Ops16 {
        Tile<bf16_t, BC, KD, NG> tk, tw, tq;
        Tile<bf16_t, BC, 16, NG> to;
        float cf;
    } opA, opB, opC;
    auto issue = [&](int ci, Ops16& o) __attribute__((always_inline)) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
        const float* R = rec + ((size_t)(slot0 + ci) * H + h) * RL::FLOATS;
        o.tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        o.tw.load(rec_w<bf16_t, KD>(R), KD, BC);
        o.tq.load(rec_qt<bf16_t, KD>(R), KD, BC);
        o.to.load(dout + (row0 * H + h) * (long)V + v0, (long)H * V, L);
        o.cf = tid < 256 ? R[RL::C_OFF + tid] : 0.f;
    };
    auto step = [&](int ci, Ops16& o) __attribute__((always_inline)) {
        if (own) {
            float* Dout = dstates + (((size_t)(slot0 + ci) * H + h) * V + v0) * KD;
#pragma unroll
            for (int r = 0; r < 4; ++r) Dout[(4 * lg + r) * KD + 16 * jc + ln] = dS[r];
            put_rows(sD, KP, 0, 16 * jc, dS);
        }
        o.tk.template store_raw<KP>(sK);
        o.tw.template store_raw<KP>(sW);
        o.tq.template store_raw<KP>(sQt);
        o.to.template store_raw<VP>(sO);
        if (tid < 256) sC[tid] = o.cf;
        __syncthreads();
        if (ci >= 3) issue(ci - 3, o);
        // Z[v][t] = e_t (dS' K^T)[v][t] on token tile w (row form), kept by token rows for the column form; with
        // it, Gamma_L dS' + dO^T Qt on the wavefront's key tile (column form: it does not wait for Z)
        if (hv == 0) {
            f32x4 Zt = mmb(sD, KP, sK + 16 * w * KP, KP, 0, KD, zero4());
            Zt = Zt * sC[128 + 16 * w + ln];
            put_cols(sZt, VP, 0, 16 * w, Zt);
        }
        f32x4 a = zero4();
        if (own) {
            a = dS * sC[64 + BC - 1];
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32) a = mma32(col8(sO, VP, k0, 0), col8(sQt, KP, k0, 16 * jc), a);
        }
        __syncthreads();
        // dS = Gamma_L dS' + dO^T Qt - Z W (column form)
        if (own) {
            f32x4 zw = zero4();
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32) zw = mma32(col8(sZt, VP, k0, 0), col8(sW, KP, k0, 16 * jc), zw);
            dS = a - zw;
        }
        __syncthreads();
    };
    if (nch > 0) issue(nch - 1, opA);
    if (nch > 1) issue(nch - 2, opB);
    if (nch > 2) issue(nch - 3, opC);
    for (int ci = nch - 1; ci >= 0; ci -= 3) {
        step(ci, opA);
        if (ci >= 1) step(ci - 1, opB);
        if (ci >= 2) step(ci - 2, opC);
    }
    if (own && dh0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) dh0[(((size_t)n * H + h) * V + v0 + 4 * lg + r) * KD + 16 * jc + ln] = dS[r];
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
        if constexpr (sizeof(ST) == 2)
            gdn_bwd_prep16_kernel<KD><<<dim3((unsigned)slots, H), 2 * NT, 0, s>>>(q, k, g, beta, table, cu, T, H, nc, scale, ws.rec);
        else
            gdn_bwd_prep_kernel<ST, KD><<<dim3((unsigned)slots, H), NT, 0, s>>>(q, k, g, beta, table, cu, T, H, nc, scale, ws.rec);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const long chains = (long)N * H;
    if (chains > 0) {
        const int nvs = V / 16;
        const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvs);
        timing_begin("gdn_bwd_states", s);
        if constexpr (sizeof(ST) == 2)
            gdn_bwd_states16_kernel<KD><<<grid, NT, 0, s>>>(k, v, h0, cu, ws.chunk_off, ws.rec, T, H, V, N, nc, nvs, ws.states);
        else
            gdn_bwd_states_kernel<ST, KD><<<grid, NT, 0, s>>>(k, v, h0, cu, ws.chunk_off, ws.rec, T, H, V, N, nc, nvs, ws.states);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        timing_begin("gdn_bwd_dstate", s);
        if constexpr (sizeof(ST) == 2)
            gdn_bwd_dstate16_kernel<KD><<<grid, 2 * NT, 0, s>>>(k, dout, dht, cu, ws.chunk_off, ws.rec, T, H, V, N, nc, nvs,
                                                            ws.dstates, dh0);
        else
            gdn_bwd_dstate_kernel<ST, KD><<<grid, NT, 0, s>>>(k, dout, dht, cu, ws.chunk_off, ws.rec, T, H, V, N, nc, nvs,
                                                              ws.dstates, dh0);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (slots > 0) {
        timing_begin("gdn_bwd_grad", s);
        if constexpr (sizeof(ST) == 2)
            gdn_bwd_grad16_kernel<KD><<<dim3((unsigned)slots, H), 2 * NT, 0, s>>>(q, k, v, dout, ws.rec, ws.states,
                                                                              ws.dstates, table, cu, T, H, V, nc, scale,
                                                                              dq, dk, dv, dg, dbeta);
        else
            gdn_bwd_grad_kernel<ST, KD><<<dim3((unsigned)slots, H), NT, 0, s>>>(q, k, v, dout, ws.rec, ws.states,
                                                                              ws.dstates, table, cu, T, H, V, nc, scale,
                                                                              dq, dk, dv, dg, dbeta);
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

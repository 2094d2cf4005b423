// Per-chunk steps of the bf16 Gated Delta Rule chunk forward, shared by its kernels.
//
// For one chunk of L <= 64 tokens of one (sequence, value head), with the within-chunk cumulative gate G,
// Gamma_t = exp(G_t), e_t = exp(G_L - G_t) and D_ti = exp(G_t - G_i) for i <= t (StateFlow Section 2.2,
// Eq. (2), Pre / ST / Out; attention-gym "Linear Attention", section "Gated Delta Rule"):
//   Pre   A = diag(beta) (strictly lower D o K K^T),  T = (I + A)^-1,  P = scale (D o Q K^T) (lower incl. diag)
//   ST    X = K S^T,  Y = V - diag(Gamma) X,  R = T diag(beta) Y,  S <- Gamma_L S + (diag(e) R)^T K
//   Out   O = scale diag(Gamma) Q S^T + P R   (S^T the chunk-entry state)
// T is formed by 16x16 blocks: the four diagonal blocks (I + A_bb)^-1 by forward substitution in float32,
// the six others from block row i of (I + A) T = I,
//   T_ij = -D_i sum_{k=j}^{i-1} A_ik T_kj   (D_j = T_jj),
// as 16x16x16 bf16 MFMA products accumulated in float32 (the page stages the solve's intermediates between
// its float32-accumulating GEMMs in the Q/K/V dtype; the solve's bf16 operands cost nothing measurable next
// to the bf16 staging of T diag(beta) itself).
//
// Every kernel of the bf16 path forms each of these with the functions below, in the same order, so a
// sequence's results do not depend on which kernel ran it or on what else shared its launch.
#pragma once

#include <type_traits>

#include "sf_device.h"
#include "sf_internal.h"

namespace sf {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) float lds_f32;

// wavefront-local order of LDS traffic: later LDS reads see the lanes' earlier writes
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// An LDS address formed in a register as it stands: the reads that follow add their constant parts in the
// instruction's offset field, instead of the compiler keeping one precomputed address per read alive.
__device__ __forceinline__ const __attribute__((address_space(3))) uint8_t* lds_base(
    const __attribute__((address_space(3))) uint8_t* p) {
    asm volatile("" : "+v"(p));
    return p;
}

// 16-byte loads of four floats and 16-byte stores, LDS or global memory
__device__ __forceinline__ f32x4 ld4(const lds_f32* p) { return *(const lds_f32x4*)p; }
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st16(lds_u8* p, u128 v) { *(__attribute__((address_space(3))) u128*)p = v; }
__device__ __forceinline__ void st16(uint8_t* p, u128 v) { *reinterpret_cast<u128*>(p) = v; }

// Fragment order of a lower-triangular 64x64 bf16 block M (T diag(beta) or P), as the MFMA operand the chain
// reads it in. Fragment f = tri_frag(ti, p) covers rows 16 ti .. 16 ti + 15 and columns 32 p .. 32 p + 31
// (p <= ti / 2, the blocks right of the diagonal tile being zero); lane (ln, lg) holds 16 bytes:
// M[16 ti + ln][32 p + 4 lg + j] then M[16 ti + ln][32 p + 16 + 4 lg + j], j = 0..3. That is the A operand of a
// 32-deep product reducing over the block's columns against a right operand made of two consecutive 16-row C
// tiles, and equally the B operand of the transposed product. Six fragments, 6 KB.
constexpr int kTriFrags = 6;
__host__ __device__ constexpr int tri_frag(int ti, int p) { return (ti == 0 ? 0 : ti == 1 ? 1 : ti == 2 ? 2 : 4) + p; }

// Per-(chunk, head) bf16 factor record of the Pre kernel: the six T diag(beta) fragments, then the 256
// coefficients [0,64) Gamma_t  [64,128) e_t  [128,192) beta_t  [192,256) G_t log2(e).
constexpr int kRecCoefOffset = kTriFrags * 1024;
static_assert(kRecCoefOffset + 1024 == kGdnRecordBf16, "record layout");

// ---------------------------------------------------------------------------------------------------------
// The natural-log gate of one token: g as given, or the gate transform of the raw per-head projection
// (attention-gym "Linear Attention", "Gate Transforms"), in float32 with the accurate exponential and log1p.
// Split into the load and the transform so that a kernel can issue the load a step ahead.
// ---------------------------------------------------------------------------------------------------------
__device__ __forceinline__ float gate_load_raw(const float* __restrict__ g, const GateSrc& gs, size_t gi) {
    if (gs.raw == nullptr) return g[gi];
    return gs.raw_bf16 ? bf2f(static_cast<const bf16_t*>(gs.raw)[gi]) : static_cast<const float*>(gs.raw)[gi];
}
// The head's transform parameters, read once: amp = exp(A_log[h]) and dt_bias[h] (unused for a given g).
struct GateHead {
    float amp, bias;
};
__device__ __forceinline__ GateHead gate_head(const GateSrc& gs, int h) {
    if (gs.raw == nullptr) return GateHead{0.f, 0.f};
    return GateHead{expf(gs.A_log[h]), gs.dt_bias[h]};
}
__device__ __forceinline__ float gate_finish(float raw, const GateSrc& gs, const GateHead& gh) {
    if (gs.raw == nullptr) return raw;
    const float x = raw + gh.bias;
    if (gs.bounded) return gs.lower_bound / (1.f + expf(-gh.amp * x));
    return -gh.amp * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))));
}

// ---------------------------------------------------------------------------------------------------------
// Solve scratch of one chunk (LDS, 9 KB), written by the first part of Pre and read by the second:
//   AOFF  the six off-diagonal 16x16 blocks A_ij of A in the order (1,0) (2,0) (2,1) (3,0) (3,1) (3,2), each
//         as its bf16 A-operand fragment (lane-major, 8 bytes per lane: A_ij[ln][4 lg + q])
//   DC    the four D_b = (I + A_bb)^-1 as bf16 C tiles (lane-major, 8 bytes per lane): D_b as a B operand
//   DTC   the four D_b^T the same way: D_b as an A operand, D_b^T as a B operand
//   TDG   the four diagonal blocks of T diag(beta) as their fragment halves: lane (ln, lg) holds
//         bf16(D_b[ln][4 lg + j] beta_{16 b + 4 lg + j}), j = 0..3
// ---------------------------------------------------------------------------------------------------------
constexpr int kSolveAoff = 0;
constexpr int kSolveDC = kSolveAoff + 6 * 256 * 2;
constexpr int kSolveDTC = kSolveDC + 4 * 512;
constexpr int kSolveTDG = kSolveDTC + 4 * 512;
constexpr int kSolveBytes = kSolveTDG + 4 * 512;
__host__ __device__ constexpr int off_blk(int i, int j) { return i * (i - 1) / 2 + j; }

// 16x16x16 bf16 MFMA: C += A B, with A given as its A-operand fragment and B as its B-operand fragment.
// A C tile X (lane (ln, lg) holds X[4 lg + j][ln]) is, packed, the B operand of X and the A operand of X^T.
__device__ __forceinline__ f32x4 mm16(i16x4 a, i16x4 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0); }

// 2^x with the hardware exponential (v_exp_f32)
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pre, gates (one wavefront, lane t = token t of the chunk): G, the inclusive gate sum (padded tokens repeat
// the last one), and the 256 coefficients [0,64) Gamma_t = exp(G_t), [64,128) e_t = exp(G_L - G_t) (hardware
// exponential; both exponents are <= 0), [128,192) beta_t (0 on padded tokens) in Pre's own copy (LDS), and in
// the record the decay from token t to the last token of its 16-token tile, w_t = exp(G_end - G_t) <= 1, which
// the off-diagonal tiles of P take (p_row), [192,256) G_t log2(e); into coef (LDS or global).
template <bool RECORD, typename CoefPtr>
__device__ __forceinline__ void pre_coefs(float G, float bv, CoefPtr coef) {
    const int lane = lane_id();
    const float GL = __shfl(G, 63, 64);
    const float G2 = G * 1.4426950408889634f;  // log2 units: every decay mask is one hardware exp2
    coef[lane] = __expf(G);
    coef[64 + lane] = __expf(GL - G);
    if constexpr (RECORD)
        coef[128 + lane] = hw_exp2(fminf(__shfl(G2, lane | 15, 64) - G2, 0.f));
    else
        coef[128 + lane] = bv;
    coef[192 + lane] = G2;
}

// Pre, first part, one half of the tiles (one wavefront): A = diag(beta) (strictly lower D o K K^T) on five of
// the ten lower 16x16 tiles (raw K K^T on 16x16x32 bf16 MFMA, then the decay mask), half 0 the tiles
// (0,0) (1,0) (1,1) (2,0) (3,0) and half 1 (2,1) (2,2) (3,1) (3,2) (3,3). Off-diagonal tiles go to AOFF. Each
// diagonal tile N = A_bb is inverted in registers by the product form
//   (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8)     (N strictly lower, so N^16 = 0)
// on bf16 MFMA, carrying every factor and its transpose (the factors are polynomials in N and commute, so a
// product and its transpose each take one MFMA from the two C tiles); D_b, D_b^T and T's diagonal block go to
// DC, DTC and TDG.
//   kf[R][p]: K row fragments of the chunk, lane (ln, lg) holding K[16 R + ln][32 p + 8 lg .. + 7]
//   cf: the chunk's coefficients (pre_coefs), of which G and beta are read
template <int HALF, int KP, typename CoefPtr>
__device__ __forceinline__ void pre_tiles(const bf16x8 (&kf)[4][KP], CoefPtr cf, lds_u8* sc) {
    typedef Elem<bf16_t> El;
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    // tile q5 of this half: (ti, tj)
    auto tile_i = [](int q5) { return HALF == 0 ? (q5 == 0 ? 0 : q5 <= 2 ? 1 : q5 == 3 ? 2 : 3) : (q5 <= 1 ? 2 : 3); };
    auto tile_j = [](int q5) { return HALF == 0 ? (q5 == 0 ? 0 : q5 == 1 ? 0 : q5 == 2 ? 1 : 0) : (q5 == 0 ? 1 : q5 == 1 ? 2 : q5 - 1); };
    // the five raw K K^T tiles first (independent accumulations). An off-diagonal tile (ti, tj) is formed
    // transposed, with K rows of block tj as the A operand: lane (ln, lg) holds (K K^T)[16 tj + 4 lg + r][16 ti + ln],
    // the element (16 ti + ln, 16 tj + 4 lg + r) of the symmetric product, so its masked values are A_ij's A-operand
    // fragment as they stand. A diagonal tile's C tile holds (K K^T)[16 ti + 4 lg + r][16 ti + ln].
    f32x4 a[5];
#pragma unroll
    for (int q5 = 0; q5 < 5; ++q5) a[q5] = zero4();
#pragma unroll
    for (int p = 0; p < KP; ++p)
#pragma unroll
        for (int q5 = 0; q5 < 5; ++q5)
            a[q5] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tile_j(q5)][p], kf[tile_i(q5)][p], a[q5], 0, 0, 0);
    // decay masks (G in log2 units); off-diagonal tiles to AOFF, the two diagonal tiles as N and N^T (C tiles):
    // element (4 lg + r, ln) of N is nonzero below the diagonal, of N^T above
    f32x4 N[2], Nt[2], bd[2];
    int nd = 0;
#pragma unroll
    for (int q5 = 0; q5 < 5; ++q5) {
        const int ti = tile_i(q5), tj = tile_j(q5);
        if (ti != tj) {
            // element (t = 16 ti + ln, s = 16 tj + 4 lg + r): beta_t 2^(G2_t - G2_s) (K K^T)_ts, t > s
            const float Gt = cf[192 + 16 * ti + ln], bt = cf[128 + 16 * ti + ln];
            const f32x4 Gs = ld4(cf + 192 + 16 * tj + 4 * lg);
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = bt * hw_exp2(fminf(Gt - Gs[r], 0.f)) * a[q5][r];
            *(lds_i16x4*)(sc + kSolveAoff + off_blk(ti, tj) * 512 + lane * 8) = El::pack(v);
        } else {
            const float Gc = cf[192 + 16 * tj + ln], bc = cf[128 + 16 * tj + ln];
            const f32x4 Gr4 = ld4(cf + 192 + 16 * ti + 4 * lg), br4 = ld4(cf + 128 + 16 * ti + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = 4 * lg + r;
                const float e = hw_exp2(fminf(Gr4[r] - Gc, Gc - Gr4[r]));  // 2^-|G2_row - G2_col|
                N[nd][r] = ln < rl ? br4[r] * e * a[q5][r] : 0.f;
                Nt[nd][r] = rl < ln ? bc * e * a[q5][r] : 0.f;
            }
            bd[nd] = br4;
            ++nd;
        }
    }
    // (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) for both diagonal blocks, interleaved. Products of
    // polynomials in N, each carried with its transpose: for commuting X and Y,
    //   C(X Y) = mm(A operand of X = pack C(X^T), B operand of Y = pack C(Y)),
    //   C((X Y)^T) = mm(A operand of Y^T = pack C(Y), B operand of X^T = pack C(X^T))
    auto prod = [&](const f32x4& Xt, const f32x4& Y, f32x4& Z, f32x4& Zt) __attribute__((always_inline)) {
        const i16x4 xt = El::pack(Xt), y = El::pack(Y);
        Z = mm16(xt, y, zero4());
        Zt = mm16(y, xt, zero4());
    };
    auto ident = [&](float sign, const f32x4& X) __attribute__((always_inline)) {  // I + sign X
        f32x4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (4 * lg + j == ln ? 1.f : 0.f) + sign * X[j];
        return r;
    };
    f32x4 N2[2], N2t[2], N4[2], N4t[2], N8[2], N8t[2], X1[2], X1t[2], X2[2], X2t[2], D[2], Dt[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) prod(Nt[d], N[d], N2[d], N2t[d]);
#pragma unroll
    for (int d = 0; d < 2; ++d) prod(N2t[d], N2[d], N4[d], N4t[d]);
#pragma unroll
    for (int d = 0; d < 2; ++d) prod(ident(-1.f, Nt[d]), ident(1.f, N2[d]), X1[d], X1t[d]);
#pragma unroll
    for (int d = 0; d < 2; ++d) prod(N4t[d], N4[d], N8[d], N8t[d]);
#pragma unroll
    for (int d = 0; d < 2; ++d) prod(X1t[d], ident(1.f, N4[d]), X2[d], X2t[d]);
#pragma unroll
    for (int d = 0; d < 2; ++d) prod(X2t[d], ident(1.f, N8[d]), D[d], Dt[d]);
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const int bb = HALF == 0 ? d : 2 + d;  // the diagonal blocks of this half
        *(lds_i16x4*)(sc + kSolveDC + bb * 512 + lane * 8) = El::pack(D[d]);
        *(lds_i16x4*)(sc + kSolveDTC + bb * 512 + lane * 8) = El::pack(Dt[d]);
        // T's diagonal block scaled by beta of its columns: lane holds D[ln][4 lg + j] = Dt's C tile element
        *(lds_i16x4*)(sc + kSolveTDG + bb * 512 + lane * 8) = El::pack(Dt[d] * bd[d]);
    }
}

// Pre, second part (one wavefront): the off-diagonal blocks of T from block row i of (I + A) T = I,
//   T_ij = -D_i U_ij,  U_ij = sum_{k=j}^{i-1} A_ik T_kj   (T_jj = D_j),
// one block diagonal i - j at a time, carrying C(T_ij) (the B operand of later products) and forming
// C(T_ij^T) = -mm(U_ij^T, D_i^T), whose lanes are already the fragment layout of T's block (ti, j); then
// T diag(beta) in fragment order (tri_frag) straight from registers.
//   beta: the chunk's 64 betas (coefficients [128, 192)); dst: the six fragments, 6 KB (LDS or global)
template <typename BetaPtr, typename DstPtr>
__device__ __forceinline__ void pre_part_t(lds_u8* sc, BetaPtr beta, DstPtr dst) {
    typedef Elem<bf16_t> El;
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    auto a_op = [&](int i, int j) __attribute__((always_inline)) {  // A_ij as A operand
        return *(const lds_i16x4*)(sc + kSolveAoff + off_blk(i, j) * 512 + lane * 8);
    };
    auto dc = [&](int b) __attribute__((always_inline)) { return *(const lds_i16x4*)(sc + kSolveDC + b * 512 + lane * 8); };
    auto dtc = [&](int b) __attribute__((always_inline)) { return *(const lds_i16x4*)(sc + kSolveDTC + b * 512 + lane * 8); };
    f32x4 Tb[4][4];   // C(T_ij), i > j
    i16x4 Fr[4][4];   // bf16 fragment halves of T diag(beta), block (i, j): lane holds T[16 i + ln][16 j + 4 lg + q] beta
#pragma unroll
    for (int dd = 1; dd < 4; ++dd)
#pragma unroll
        for (int j = 0; j + dd < 4; ++j) {
            const int i = j + dd;
            f32x4 uu = mm16(a_op(i, j), dc(j), zero4());
#pragma unroll
            for (int kk = j + 1; kk < i; ++kk) uu = mm16(a_op(i, kk), El::pack(Tb[kk][j]), uu);
            const i16x4 up = El::pack(uu), dti = dtc(i);
            Tb[i][j] = mm16(dti, up, zero4()) * -1.f;                 // C(T_ij) = -C(D_i U)
            const f32x4 tt = mm16(up, dti, zero4()) * -1.f;            // C(T_ij^T) = -C(U^T D_i^T)
            const f32x4 bcol = ld4(beta + 16 * j + 4 * lg);
            Fr[i][j] = El::pack(tt * bcol);
        }
#pragma unroll
    for (int b = 0; b < 4; ++b) Fr[b][b] = *(const lds_i16x4*)(sc + kSolveTDG + b * 512 + lane * 8);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int p = 0; p <= ti / 2; ++p) {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            const i16x4 z = {0, 0, 0, 0};
            const u32x2 lo = __builtin_bit_cast(u32x2, Fr[ti][2 * p]);
            const u32x2 hi = __builtin_bit_cast(u32x2, 2 * p + 1 <= ti ? Fr[ti][2 * p + 1] : z);
            st16(dst + (tri_frag(ti, p) * 64 + lane) * 16, u128{lo[0], lo[1], hi[0], hi[1]});
        }
}

// The whole of Pre in one wavefront (the Pre kernel): coefficients (into the LDS block scf, which the tiles
// read, and to coef), both halves of the tiles, the solve.
template <int KP, typename CoefPtr, typename DstPtr>
__device__ __forceinline__ void pre_all(const bf16x8 (&kf)[4][KP], float G, float bv, lds_f32* scf, CoefPtr coef,
                                        lds_u8* sc, DstPtr dst) {
    pre_coefs<false>(G, bv, scf);
    pre_coefs<true>(G, bv, coef);
    wave_lds_sync();
    pre_tiles<0, KP>(kf, scf, sc);
    pre_tiles<1, KP>(kf, scf, sc);
    wave_lds_sync();
    pre_part_t(sc, scf + 128, dst);
}

// ---------------------------------------------------------------------------------------------------------
// Block row TI of P^T = scale (D o Q K^T)^T in registers: kf[tj][p] the K row fragments of token tiles
// tj <= TI, qf[p] the Q row fragments of token tile TI; pf[p], p <= TI / 2, gets fragment (TI, p)'s lane
// content. P^T tiles with K rows as A (rows s) and Q rows as B (columns t): the C tile holds, for lane (ln, lg),
// P[16 TI + ln][16 tj + 4 lg + r], which is fragment (TI, tj / 2)'s lane content (first or second half), the B
// operand that pairs with the R fragments of the same tokens. cf: the record's coefficients (G in log2 units
// at [192, 256), w at [128, 192)). The decay exp(G_t - G_s) of a diagonal tile is one exponential per element;
// an off-diagonal tile (s in an earlier tile tj) splits it at the last token e of tile tj into exp(G_t - G_e)
// per row and w_s = exp(G_e - G_s) per column, both <= 1, so neither factor overflows where the product is
// finite.
// ---------------------------------------------------------------------------------------------------------
template <int TI, int KP>
__device__ __forceinline__ void p_row(const bf16x8 (&kf)[4][KP], const bf16x8 (&qf)[KP], const lds_f32* cf, float scale,
                                      bf16x8 (&pf)[2]) {
    typedef Elem<bf16_t> El;
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    const float Gt = cf[192 + 16 * TI + ln];
    f32x4 PT[4];
#pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
        PT[tj] = zero4();
        if (tj <= TI) {
#pragma unroll
            for (int p = 0; p < KP; ++p) PT[tj] = mma32(kf[tj][p], qf[p], PT[tj]);
        }
    }
#pragma unroll
    for (int tj = 0; tj < TI; ++tj) {
        const float a = scale * hw_exp2(fminf(Gt - cf[192 + 16 * tj + 15], 0.f));
        const f32x4 w = *(const lds_f32x4*)(cf + 128 + 16 * tj + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) PT[tj][r] = PT[tj][r] * a * w[r];
    }
    {
        const f32x4 Gs = *(const lds_f32x4*)(cf + 192 + 16 * TI + 4 * lg);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            // token s = 16 TI + 4 lg + r against t = 16 TI + ln: only s <= t, where G_t - G_s <= 0
            const bool keep = 4 * lg + r <= ln;
            PT[TI][r] = keep ? PT[TI][r] * (scale * hw_exp2(fminf(Gt - Gs[r], 0.f))) : 0.f;
        }
    }
#pragma unroll
    for (int p = 0; p <= TI / 2; ++p) pf[p] = cat8(El::pack(PT[2 * p]), El::pack(PT[2 * p + 1]));
}

// P of one chunk from the K and Q rows in LDS (RowBlock layout) into LDS in fragment order, for the block rows
// set in ROWS (bit ti: block row ti), each row by p_row.
template <int KD, int ROWS>
__device__ __forceinline__ void form_p(const lds_u8* KR, const lds_u8* QR, const lds_f32* cf, float scale, lds_u8* P) {
    typedef RowBlock<KD> RBk;
    constexpr int KP = KD / 32;
    constexpr int UST = (16 / RBk::RPB) * 1024;
    constexpr int TOP = (ROWS & 8) ? 3 : (ROWS & 4) ? 2 : (ROWS & 2) ? 1 : 0;  // highest block row formed
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    int orow[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p) orow[p] = RBk::off(ln, 4 * p + lg);
    bf16x8 kf[4][KP];
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int p = 0; p < KP; ++p)
            if (R <= TOP) kf[R][p] = *(const lds_bf16x8*)(KR + orow[p] + R * UST);
    auto row = [&](auto ti_c) __attribute__((always_inline)) {
        constexpr int ti = decltype(ti_c)::value;
        if constexpr ((ROWS >> ti) & 1) {
            bf16x8 qf[KP], pf[2];
#pragma unroll
            for (int p = 0; p < KP; ++p) qf[p] = *(const lds_bf16x8*)(QR + orow[p] + ti * UST);
            p_row<ti, KP>(kf, qf, cf, scale, pf);
#pragma unroll
            for (int p = 0; p <= ti / 2; ++p) *(lds_bf16x8*)(P + tri_frag(ti, p) * 1024 + lane * 16) = pf[p];
        }
    };
    row(std::integral_constant<int, 0>{});
    row(std::integral_constant<int, 1>{});
    row(std::integral_constant<int, 2>{});
    row(std::integral_constant<int, 3>{});
}

// ---------------------------------------------------------------------------------------------------------
// One 16-row state slice's chunk step. State tiles: S[kt], kt = 2 p + hh, is the C tile of S^T whose row
// 4 lg + j stands for key column 32 p + 8 lg + 4 hh + j and whose column ln for state row row0 + ln; the pair
// (S[2p], S[2p+1]) gives lane group lg the eight consecutive columns 32 p + 8 lg .. + 7, so K and Q rows enter
// the products as plain 16-byte row fragments (RowBlock layout in LDS).
// ---------------------------------------------------------------------------------------------------------
template <int KD>
struct SliceOps {
    typedef RowBlock<KD> RBk;
    typedef Elem<bf16_t> El;
    static constexpr int KP = KD / 32, KB = KD / 16;
    static constexpr int UST = (16 / RBk::RPB) * 1024;  // byte step of one 16-row token tile in a row block

    __device__ static int orow(int p) { return RBk::off(lane_id() & 15, 4 * p + (lane_id() >> 4)); }
    __device__ static int otr(int p) {
        const int ln = lane_id() & 15, lg = lane_id() >> 4;
        return RBk::off(4 * lg + (ln >> 2), 4 * p + (ln & 3));
    }

    // The residual, by halves over the token tiles: for the token tiles U0, U0 + 1, x_in issues the LDS reads
    // (K row fragments, the Gamma coefficients, the V block) and x_mul forms X = K S^T from the bf16 entry state
    // Sf; residual_yx forms Y = V - Gamma X in bf16. KR: K rows; vtr: this slice's V block [64][16] bf16 at the
    // lane's transposed-read offset; cf: coefficients. The two schedules below (residual, residual_split) make
    // the same products in the same order, so they give the same bits.
    template <int U0>
    struct XIn {
        bf16x8 kr[2][KP];
        f32x4 gam[2];
        i16x4 vx[2];
    };
    template <int U0>
    struct XOut {
        f32x4 X[2], gam[2];
        i16x4 vx[2];
    };
    template <int U0>
    __device__ static XIn<U0> x_in(const lds_u8* KR, const lds_u8* vtr, const lds_f32* cf) {
        const int lg = lane_id() >> 4;
        XIn<U0> in;
#pragma unroll
        for (int p = 0; p < KP; ++p) {
            const lds_u8* kb = lds_base(KR + orow(p));
#pragma unroll
            for (int u = 0; u < 2; ++u) in.kr[u][p] = *(const lds_bf16x8*)(kb + (U0 + u) * UST);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            in.gam[u] = *(const lds_f32x4*)(cf + 16 * (U0 + u) + 4 * lg);
            in.vx[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vtr + 16 * (U0 + u) * 16 * 2));
        }
        return in;
    }
    // X = K S^T on the two token tiles from their K row fragments kr (the two tiles' accumulations interleaved,
    // each summed over p in order)
    __device__ static void x_prod(const bf16x8 (&kr)[2][KP], const i16x4 (&Sf)[KB], f32x4 (&X)[2]) {
        X[0] = zero4();
        X[1] = zero4();
#pragma unroll
        for (int p = 0; p < KP; ++p)
#pragma unroll
            for (int u = 0; u < 2; ++u) X[u] = mma32(kr[u][p], cat8(Sf[2 * p], Sf[2 * p + 1]), X[u]);
    }
    template <int U0>
    __device__ static XOut<U0> x_mul(const XIn<U0>& in, const i16x4 (&Sf)[KB]) {
        XOut<U0> o;
        x_prod(in.kr, Sf, o.X);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            o.gam[u] = in.gam[u];
            o.vx[u] = in.vx[u];
        }
        return o;
    }
    // reads, then products (the reads' latency paid once per half)
    template <int U0>
    __device__ static XOut<U0> residual_x(const i16x4 (&Sf)[KB], const lds_u8* KR, const lds_u8* vtr, const lds_f32* cf) {
        const XIn<U0> in = x_in<U0>(KR, vtr, cf);
        __builtin_amdgcn_sched_barrier(0);
        return x_mul<U0>(in, Sf);
    }
    // Y = V - Gamma X on those tiles in bf16; vmask zeroes V for transition rows
    template <int U0>
    __device__ static void residual_yx(const XOut<U0>& x, uint32_t vmask, i16x4 (&Yf)[2]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
            const i16x4 Vf = __builtin_bit_cast(i16x4, __builtin_bit_cast(u32x2, x.vx[u]) & vmask);
            Yf[u] = El::pack(El::unpack(Vf) - x.gam[u] * x.X[u]);
        }
    }
    // The T diag(beta) fragments and the e coefficients that residual_r<U0> needs (they do not depend on Y):
    // fragments (U0, 0) and (U0 + 1, 0), and for U0 = 2 also (2, 1), (3, 1). Tfr: the six fragments.
    template <int U0>
    struct RIn {
        bf16x8 tf[U0 == 0 ? 2 : 4];
        f32x4 ec[2];
    };
    __device__ static bf16x8 tri_in(const lds_u8* Tfr, int ti, int p) {
        return *(const lds_bf16x8*)(Tfr + tri_frag(ti, p) * 1024 + lane_id() * 16);
    }
    template <int U0>
    __device__ static RIn<U0> residual_r_in(const lds_f32* cf, const lds_u8* Tfr) {
        const int lg = lane_id() >> 4;
        RIn<U0> in;
        auto tf = [&](int ti, int p) __attribute__((always_inline)) { return tri_in(Tfr, ti, p); };
        if constexpr (U0 == 0) {
            in.tf[0] = tf(0, 0);
            in.tf[1] = tf(1, 0);
        } else {
            in.tf[0] = tf(2, 0);
            in.tf[1] = tf(2, 1);
            in.tf[2] = tf(3, 0);
            in.tf[3] = tf(3, 1);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) in.ec[i] = *(const lds_f32x4*)(cf + 64 + 16 * (U0 + i) + 4 * lg);
        return in;
    }
    // residual_r<U0>: R = T diag(beta) Y on the token tiles U0, U0 + 1 (T lower triangular: tiles 0 and 1 need
    // Y of tiles 0, 1 only, as Y01; tiles 2 and 3 also Y23), and ER = e o R in bf16.
    template <int U0>
    __device__ static void residual_r(bf16x8 Y01, bf16x8 Y23, const RIn<U0>& in, f32x4 (&R)[2], i16x4 (&ER)[2]) {
        if constexpr (U0 == 0) {
            R[0] = mma32(in.tf[0], Y01, zero4());
            R[1] = mma32(in.tf[1], Y01, zero4());
        } else {
            R[0] = mma32(in.tf[1], Y23, mma32(in.tf[0], Y01, zero4()));
            R[1] = mma32(in.tf[3], Y23, mma32(in.tf[2], Y01, zero4()));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) ER[i] = El::pack(R[i] * in.ec[i]);
    }
    // R = T diag(beta) (V - diag(Gamma) K S^T) from the bf16 entry state Sf; ER = e o R in bf16.
    // residual: one half after the other, for callers short of registers.
    __device__ static void residual(const i16x4 (&Sf)[KB], const lds_u8* KR, const lds_u8* vtr, uint32_t vmask,
                                    const lds_f32* cf, const lds_u8* Tfr, f32x4 (&R)[4], i16x4 (&ER)[4]) {
        const RIn<0> in0 = residual_r_in<0>(cf, Tfr);
        const RIn<2> in2 = residual_r_in<2>(cf, Tfr);
        i16x4 Ylo[2], Yhi[2];
        residual_yx<0>(residual_x<0>(Sf, KR, vtr, cf), vmask, Ylo);
        residual_yx<2>(residual_x<2>(Sf, KR, vtr, cf), vmask, Yhi);
        residual_ry(Ylo, Yhi, in0, in2, R, ER);
    }
    // residual_split: the schedule of one wavefront that runs the whole step. The LDS reads return in order and
    // the wait counter reaches back 15 reads only, so the reads go out in the order of their use, each batch
    // behind products that cover its latency: the K row fragments of all four tiles (first() issues a caller's
    // early reads ahead of them), the first half's products, the Gamma, V, T diag(beta) and e reads, the second
    // half's products, after_x() (a caller's reads and arithmetic that need none of these), Y, after_y(), R.
    template <typename First, typename AfterX, typename AfterY>
    __device__ static void residual_split(const i16x4 (&Sf)[KB], const lds_u8* KR, const lds_u8* vtr, uint32_t vmask,
                                          const lds_f32* cf, const lds_u8* Tfr, f32x4 (&R)[4], i16x4 (&ER)[4],
                                          First&& first, AfterX&& after_x, AfterY&& after_y) {
        const int lg = lane_id() >> 4;
        first();
        bf16x8 kr0[2][KP], kr2[2][KP];
#pragma unroll
        for (int p = 0; p < KP; ++p) {
            const lds_u8* kb = lds_base(KR + orow(p));
#pragma unroll
            for (int u = 0; u < 2; ++u) kr0[u][p] = *(const lds_bf16x8*)(kb + u * UST);
        }
#pragma unroll
        for (int p = 0; p < KP; ++p) {
            const lds_u8* kb = lds_base(KR + orow(p));
#pragma unroll
            for (int u = 0; u < 2; ++u) kr2[u][p] = *(const lds_bf16x8*)(kb + (2 + u) * UST);
        }
        __builtin_amdgcn_sched_barrier(0);
        XOut<0> x0;
        XOut<2> x2;
        x_prod(kr0, Sf, x0.X);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 gam = *(const lds_f32x4*)(cf + 16 * u + 4 * lg);
            const i16x4 vx = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vtr + 16 * u * 16 * 2));
            if (u < 2) {
                x0.gam[u] = gam;
                x0.vx[u] = vx;
            } else {
                x2.gam[u - 2] = gam;
                x2.vx[u - 2] = vx;
            }
        }
        const RIn<0> in0 = residual_r_in<0>(cf, Tfr);
        const RIn<2> in2 = residual_r_in<2>(cf, Tfr);
        __builtin_amdgcn_sched_barrier(0);
        x_prod(kr2, Sf, x2.X);
        __builtin_amdgcn_sched_barrier(0);
        after_x();
        __builtin_amdgcn_sched_barrier(0);
        i16x4 Ylo[2], Yhi[2];
        residual_yx<0>(x0, vmask, Ylo);
        residual_yx<2>(x2, vmask, Yhi);
        __builtin_amdgcn_sched_barrier(0);
        after_y();
        __builtin_amdgcn_sched_barrier(0);
        residual_ry(Ylo, Yhi, in0, in2, R, ER);
    }
    __device__ static void residual_ry(const i16x4 (&Ylo)[2], const i16x4 (&Yhi)[2], const RIn<0>& in0,
                                       const RIn<2>& in2, f32x4 (&R)[4], i16x4 (&ER)[4]) {
        const bf16x8 Y01 = cat8(Ylo[0], Ylo[1]), Y23 = cat8(Yhi[0], Yhi[1]);
        f32x4 Rlo[2], Rhi[2];
        i16x4 Elo[2], Ehi[2];
        residual_r<0>(Y01, Y23, in0, Rlo, Elo);
        residual_r<2>(Y01, Y23, in2, Rhi, Ehi);
        R[0] = Rlo[0];
        R[1] = Rlo[1];
        R[2] = Rhi[0];
        R[3] = Rhi[1];
        ER[0] = Elo[0];
        ER[1] = Elo[1];
        ER[2] = Ehi[0];
        ER[3] = Ehi[1];
    }

    // S^T <- Gamma_L S^T + K^T (e R) on the key tiles [KT0, KT0 + NKT) (S holds those tiles)
    // (split into the K^T reads, which do not depend on e R, and the products)
    template <int KT0, int NKT>
    __device__ static void read_kt(const lds_u8* KR, i16x4 (&Ka)[NKT][4]) {
#pragma unroll
        for (int i = 0; i < NKT; ++i) {
            const int kt = KT0 + i;
            const int p = kt >> 1, hh = kt & 1;
            const lds_u8* kb = lds_base(KR + otr(p));
#pragma unroll
            for (int u = 0; u < 4; ++u)
                Ka[i][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(kb + 8 * hh + u * UST));
        }
    }
    template <int NKT>
    __device__ static void update_with(f32x4 (&S)[NKT], const i16x4 (&ER)[4], const i16x4 (&Ka)[NKT][4], float gl) {
        const bf16x8 E01 = cat8(ER[0], ER[1]), E23 = cat8(ER[2], ER[3]);
        f32x4 acc[NKT];
#pragma unroll
        for (int i = 0; i < NKT; ++i) acc[i] = mma32(cat8(Ka[i][0], Ka[i][1]), E01, S[i] * gl);
#pragma unroll
        for (int i = 0; i < NKT; ++i) S[i] = mma32(cat8(Ka[i][2], Ka[i][3]), E23, acc[i]);
    }
    // the same, with the K^T fragments of the first and second half of the key tiles in Ka and Kb
    template <int NKT>
    __device__ static void update_halves(f32x4 (&S)[NKT], const i16x4 (&ER)[4], const i16x4 (&Ka)[NKT / 2][4],
                                         const i16x4 (&Kb)[NKT / 2][4], float gl) {
        const bf16x8 E01 = cat8(ER[0], ER[1]), E23 = cat8(ER[2], ER[3]);
        auto kf = [&](int i, int u) __attribute__((always_inline)) { return i < NKT / 2 ? Ka[i][u] : Kb[i - NKT / 2][u]; };
        f32x4 acc[NKT];
#pragma unroll
        for (int i = 0; i < NKT; ++i) acc[i] = mma32(cat8(kf(i, 0), kf(i, 1)), E01, S[i] * gl);
#pragma unroll
        for (int i = 0; i < NKT; ++i) S[i] = mma32(cat8(kf(i, 2), kf(i, 3)), E23, acc[i]);
    }
    template <int KT0, int NKT>
    __device__ static void update_tiles(f32x4 (&S)[NKT], const i16x4 (&ER)[4], const lds_u8* KR, float gl) {
        i16x4 Ka[NKT][4];
        read_kt<KT0, NKT>(KR, Ka);
        update_with<NKT>(S, ER, Ka, gl);
    }

    // S^T <- Gamma_L S^T + K^T (e R)
    __device__ static void update(f32x4 (&S)[KB], const i16x4 (&ER)[4], const lds_u8* KR, float gl) {
        update_tiles<0, KB>(S, ER, KR, gl);
    }

    // O^T tile tt (16 tokens) of the slice: scale Gamma (S Q^T) + R^T P^T, from the bf16 entry state Sf, the
    // bf16 corrected values Rb, Q row fragments qf[p] of the tile, gq = Gamma_t scale of the lane's token and
    // the P fragments of block row tt (pf[pp], pp <= tt / 2). Lane (ln, lg) gets o[16 tt + ln][row0 + 4 lg + j].
    __device__ static f32x4 out_tile(int tt, const i16x4 (&Sf)[KB], const i16x4 (&Rb)[4], const bf16x8 (&qf)[KP],
                                     float gq, const bf16x8 (&pf)[2]) {
        f32x4 o = zero4();
#pragma unroll
        for (int p = 0; p < KP; ++p) o = mma32(cat8(Sf[2 * p], Sf[2 * p + 1]), qf[p], o);
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
            if (pp <= tt / 2) o = mma32(cat8(Rb[2 * pp], Rb[2 * pp + 1]), pf[pp], pp == 0 ? o * gq : o);
        return o;
    }
};

}  // namespace sf

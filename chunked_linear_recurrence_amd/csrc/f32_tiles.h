// Float32 tile helpers shared by the 256-thread chunk kernels that compute in float32 (the delta-rule chunk
// backward and the Kimi Delta Attention chunk forward): 16-byte staged tile loads into padded LDS rows, and one
// 16x16 float32 MFMA tile over LDS operands.
#pragma once

#include "sf_device.h"

namespace sf {
namespace f32t {

constexpr int NT = 256;  // threads per workgroup of the kernels that use these helpers

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
// chunk's tiles while it computes on the current ones. NTH threads share the pieces.
template <typename ST, int ROWS, int COLS, int NTH = NT>
struct Tile {
    static constexpr int E = 16 / (int)sizeof(ST);
    static constexpr int PPR = COLS / E;                     // pieces per row
    static constexpr int PIECES = ROWS * PPR;
    static constexpr int PER = (PIECES + NTH - 1) / NTH;
    static_assert(COLS % E == 0, "tile rows are whole 16-byte pieces");
    u128 r[PER];
    __device__ __forceinline__ void load(const ST* __restrict__ base, long ld, int rows_valid) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = threadIdx.x + NTH * p, row = idx / PPR, col = (idx % PPR) * E;
            r[p] = u128{0u, 0u, 0u, 0u};
            if (idx < PIECES && row < rows_valid) r[p] = *reinterpret_cast<const u128*>(base + row * ld + col);
        }
    }
    // into rows of stride lds (default COLS + 1)
    __device__ __forceinline__ void store(float* dst, int lds = COLS + 1) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = threadIdx.x + NTH * p, row = idx / PPR, col = (idx % PPR) * E;
            if (idx < PIECES)
#pragma unroll
                for (int e = 0; e < E; ++e) dst[row * lds + col + e] = Elem<ST>::to_f(unit_of<ST>(r[p], e));
        }
    }
    // the pieces as they are (no conversion) into rows of stride LDS elements of ST, a multiple of 16 bytes
    template <int LDS>
    __device__ __forceinline__ void store_raw(ST* dst) const {
        static_assert(LDS * sizeof(ST) % 16 == 0, "16-byte row starts");
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = threadIdx.x + NTH * p, row = idx / PPR, col = (idx % PPR) * E;
            if (idx < PIECES) *reinterpret_cast<u128*>(dst + row * LDS + col) = r[p];
        }
    }
    // into rows of stride LDS, a multiple of four floats (dst 16-byte aligned): 16-byte LDS writes
    template <int LDS>
    __device__ __forceinline__ void store_rows(float* dst) const {
        static_assert(LDS % 4 == 0, "16-byte row starts");
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = threadIdx.x + NTH * p, row = idx / PPR, col = (idx % PPR) * E;
            if (idx < PIECES)
#pragma unroll
                for (int e = 0; e < E; e += 4) {
                    f32x4 f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) f[i] = Elem<ST>::to_f(unit_of<ST>(r[p], e + i));
                    *reinterpret_cast<f32x4*>(dst + row * LDS + col + e) = f;
                }
        }
    }
};

// Float32 MFMA tile over LDS operands: acc += A(i, k) B(k, j) for one 16x16 tile, k in [k0, k1) (a multiple of 4
// apart), with A(i, k) = A[i * ars + k * acs] and B(k, j) = B[k * brs + j * bcs] (pointers at the tile origin;
// the strides give transposed reads for free). Lane (ln, lg) brings A(ln, k + lg) times as (the scale of its A
// row) and B(k + lg, ln); the C tile holds rows 4 lg + r, column ln (v_mfma_f32_16x16x4_f32). The reads of 32
// (then 16, then 4) reduction steps are issued together before their products, so that one LDS latency
// serves several products; the products accumulate in k order either way.
__device__ __forceinline__ f32x4 mm4(const float* A, int ars, int acs, const float* B, int brs, int bcs, int k0, int k1,
                                     f32x4 acc, float as = 1.f) {
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    const float* a = A + ln * ars + lg * acs;
    const float* b = B + lg * brs + ln * bcs;
    int kk = k0;
    for (; kk + 32 <= k1; kk += 32) {
        float av[8], bv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            av[u] = a[(kk + 4 * u) * acs];
            bv[u] = b[(kk + 4 * u) * brs];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as * av[u], bv[u], acc, 0, 0, 0);
    }
    if (kk + 16 <= k1) {
        float av[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            av[u] = a[(kk + 4 * u) * acs];
            bv[u] = b[(kk + 4 * u) * brs];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as * av[u], bv[u], acc, 0, 0, 0);
        kk += 16;
    }
    for (; kk < k1; kk += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as * a[kk * acs], b[kk * brs], acc, 0, 0, 0);
    return acc;
}

// The same tile product with bf16 operands (float32 accumulation): the float32 LDS operands are rounded to bf16
// in registers, 32 reduction steps per v_mfma_f32_16x16x32_bf16 (lane (ln, lg) brings A(ln, k + 8 lg + j) and
// B(k + 8 lg + j, ln), j = 0..7) and a last 16 by v_mfma_f32_16x16x16_bf16 (A(ln, k + 4 lg + j), j = 0..3). The
// C tile layout is mm4's. k1 - k0 is a multiple of 16.
__device__ __forceinline__ f32x4 mm32(const float* A, int ars, int acs, const float* B, int brs, int bcs, int k0,
                                      int k1, f32x4 acc, float as = 1.f) {
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    const float* a = A + ln * ars;
    const float* b = B + ln * bcs;
    int kk = k0;
    for (; kk + 64 <= k1; kk += 64) {
        f32x8 av[2], bv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                av[u][j] = a[(kk + 32 * u + 8 * lg + j) * acs];
                bv[u][j] = b[(kk + 32 * u + 8 * lg + j) * brs];
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_convertvector(av[u] * as, bf16x8),
                                                          __builtin_convertvector(bv[u], bf16x8), acc, 0, 0, 0);
    }
    if (kk + 32 <= k1) {
        f32x8 av, bv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            av[j] = a[(kk + 8 * lg + j) * acs];
            bv[j] = b[(kk + 8 * lg + j) * brs];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_convertvector(av * as, bf16x8),
                                                      __builtin_convertvector(bv, bf16x8), acc, 0, 0, 0);
        kk += 32;
    }
    if (kk + 16 <= k1) {
        f32x4 av, bv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            av[j] = a[(kk + 4 * lg + j) * acs];
            bv[j] = b[(kk + 4 * lg + j) * brs];
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Elem<bf16_t>::pack(av * as), Elem<bf16_t>::pack(bv), acc, 0, 0, 0);
    }
    return acc;
}

// bf16 tile product from bf16 LDS operands: acc += A(i, k) B(k, j), A row-major (A[i * lda + k]) and B given by
// its transpose (Bt[j * ldb + k]); k in [k0, k1), k1 - k0 a multiple of 16, lda and ldb multiples of 8. Lane
// (ln, lg) reads 8 consecutive k of its A row and of its Bt row with one 16-byte read each.
__device__ __forceinline__ f32x4 mmb(const bf16_t* A, int lda, const bf16_t* Bt, int ldb, int k0, int k1, f32x4 acc) {
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    const bf16_t* a = A + ln * lda;
    const bf16_t* b = Bt + ln * ldb;
    int kk = k0;
    for (; kk + 32 <= k1; kk += 32)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(a + kk + 8 * lg),
                                                      *reinterpret_cast<const bf16x8*>(b + kk + 8 * lg), acc, 0, 0, 0);
    if (kk + 16 <= k1)
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(*reinterpret_cast<const i16x4*>(a + kk + 4 * lg),
                                                        *reinterpret_cast<const i16x4*>(b + kk + 4 * lg), acc, 0, 0, 0);
    return acc;
}

// Eight (four) elements p[0], p[stride], ... as bf16: float elements rounded to nearest even, bf16 elements as
// they are.
__device__ __forceinline__ bf16x8 bf8_of(const float* p, int stride) {
    typedef float f32x8 __attribute__((ext_vector_type(8)));
    f32x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = p[j * stride];
    return __builtin_convertvector(v, bf16x8);
}
__device__ __forceinline__ bf16x8 bf8_of(const bf16_t* p, int stride) {
    i16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (short)p[j * stride];
    return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ i16x4 bf4_of(const float* p, int stride) {
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = p[j * stride];
    return Elem<bf16_t>::pack(v);
}
__device__ __forceinline__ i16x4 bf4_of(const bf16_t* p, int stride) {
    i16x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (short)p[j * stride];
    return v;
}

// mm32 (unscaled) with each operand in LDS as float or as bf16: for the same operand values, the same products in
// the same order, so the same bits.
template <typename TA, typename TB>
__device__ __forceinline__ f32x4 mmg(const TA* A, int ars, int acs, const TB* B, int brs, int bcs, int k0, int k1,
                                     f32x4 acc) {
    const int lane = lane_id(), ln = lane & 15, lg = lane >> 4;
    const TA* a = A + ln * ars;
    const TB* b = B + ln * bcs;
    int kk = k0;
    for (; kk + 32 <= k1; kk += 32)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf8_of(a + (kk + 8 * lg) * acs, acs),
                                                      bf8_of(b + (kk + 8 * lg) * brs, brs), acc, 0, 0, 0);
    if (kk + 16 <= k1)
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bf4_of(a + (kk + 4 * lg) * acs, acs),
                                                        bf4_of(b + (kk + 4 * lg) * brs, brs), acc, 0, 0, 0);
    return acc;
}

// The tile product in the arithmetic of the input type ST: float32 operands for float32 inputs, bf16 operands
// for bf16 inputs.
template <typename ST>
__device__ __forceinline__ f32x4 mmx(const float* A, int ars, int acs, const float* B, int brs, int bcs, int k0, int k1,
                                     f32x4 acc, float as = 1.f) {
    if constexpr (sizeof(ST) == 2)
        return mm32(A, ars, acs, B, brs, bcs, k0, k1, acc, as);
    else
        return mm4(A, ars, acs, B, brs, bcs, k0, k1, acc, as);
}

}  // namespace f32t
}  // namespace sf

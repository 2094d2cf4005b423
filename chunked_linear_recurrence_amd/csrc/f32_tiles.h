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
    // into rows of stride lds (default COLS + 1)
    __device__ __forceinline__ void store(float* dst, int lds = COLS + 1) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = threadIdx.x + NT * p, row = idx / PPR, col = (idx % PPR) * E;
            if (idx < PIECES)
#pragma unroll
                for (int e = 0; e < E; ++e) dst[row * lds + col + e] = Elem<ST>::to_f(unit_of<ST>(r[p], e));
        }
    }
    // into rows of stride LDS, a multiple of four floats (dst 16-byte aligned): 16-byte LDS writes
    template <int LDS>
    __device__ __forceinline__ void store_rows(float* dst) const {
        static_assert(LDS % 4 == 0, "16-byte row starts");
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int idx = threadIdx.x + NT * p, row = idx / PPR, col = (idx % PPR) * E;
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

}  // namespace f32t
}  // namespace sf

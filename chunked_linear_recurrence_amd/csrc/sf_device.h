// Device-side building blocks for the gfx950 kernels: element types, the
// 16x16 MFMA block product, LDS fragment loads and bf16 conversion.
//
// Block product convention (one 64-lane wavefront):
//   lane = 16 * lg + ln  (ln in 0..15, lg in 0..3)
//   A fragment of a 16x16 block A[m][r]:  lane holds A[ln][4*lg + j], j = 0..3
//   B fragment of a 16x16 block B[r][n]:  lane holds B[4*lg + j][ln], j = 0..3
//   C/D tile of a 16x16 block C[m][n]:    lane holds C[4*lg + j][ln], j = 0..3
// so the C tile of one product is, unchanged, the B fragment of a product
// that reduces over the C tile's row index, and (as C^T) the A fragment of a
// product whose rows are the C tile's columns. For bf16 storage one block
// product is one v_mfma_f32_16x16x16_bf16; for float32 it is four
// v_mfma_f32_16x16x4_f32 issued over the four reduction slots j.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sf {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// float32 -> bf16 with the hardware converter (v_cvt_pk_bf16_f32: round to
// nearest even, NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

template <typename ST> struct Elem;

template <> struct Elem<bf16_t> {
    typedef i16x4 frag;
    static __device__ __forceinline__ float to_f(bf16_t x) { return bf2f(x); }
    static __device__ __forceinline__ bf16_t from_f(float x) { return f2bf(x); }
    static __device__ __forceinline__ f32x4 mma(f32x4 acc, frag a, frag b) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
    }
    // Two consecutive 16-wide reduction blocks in one v_mfma_f32_16x16x32_bf16:
    // lane slots 0..3 carry block 0 and 4..7 block 1 in both operands, so the
    // 32 products pair up exactly as in two block products.
    static __device__ __forceinline__ f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
        const i16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        const i16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       acc, 0, 0, 0);
    }
    // float32 -> bf16 with the hardware converter (v_cvt_pk_bf16_f32, round to
    // nearest even), two values per instruction. Converted as two 2-wide vectors:
    // a 4-wide conversion is sometimes split into one value per instruction plus
    // byte permutes (three times the instructions, in the chain's step too).
    static __device__ __forceinline__ frag pack(f32x4 x) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const bf16x2 lo = __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2);
        const bf16x2 hi = __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2);
        return __builtin_bit_cast(frag, u32x2{__builtin_bit_cast(unsigned int, lo), __builtin_bit_cast(unsigned int, hi)});
    }
    static __device__ __forceinline__ f32x4 unpack(frag x) {
        f32x4 r;
        r[0] = bf2f((bf16_t)x[0]);
        r[1] = bf2f((bf16_t)x[1]);
        r[2] = bf2f((bf16_t)x[2]);
        r[3] = bf2f((bf16_t)x[3]);
        return r;
    }
};

template <> struct Elem<float> {
    typedef f32x4 frag;
    static __device__ __forceinline__ float to_f(float x) { return x; }
    static __device__ __forceinline__ float from_f(float x) { return x; }
    static __device__ __forceinline__ f32x4 mma(f32x4 acc, frag a, frag b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
        return acc;
    }
    static __device__ __forceinline__ f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
        return mma(mma(acc, a0, b0), a1, b1);
    }
    static __device__ __forceinline__ frag pack(f32x4 x) { return x; }
    static __device__ __forceinline__ f32x4 unpack(frag x) { return x; }
};

// Fragment of rows [r0, r0+16) x columns [c0 + 4*lg, +4) of a row-major
// LDS matrix with leading dimension ld. Serves as the A fragment of
// X[r0.., c0..] and as the B fragment of (Y[r0.., c0..])^T.
template <typename ST>
__device__ __forceinline__ typename Elem<ST>::frag frag_rows(const ST* m, int ld, int r0, int c0) {
    const int ln = lane_id() & 15, lg = lane_id() >> 4;
    return *reinterpret_cast<const typename Elem<ST>::frag*>(m + (r0 + ln) * ld + c0 + 4 * lg);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16-byte vector unit used for staging copies. A native vector type (not
// HIP's uint4 struct, whose copies become stack memcpys) so that staging
// values stay in registers.
typedef unsigned int u128 __attribute__((ext_vector_type(4)));

// Inclusive prefix sum over the 64 lanes of a wavefront, on DPP lane moves: within each row of 16 lanes by
// shifts of 1, 2, 4 and 8, then the last lane of row 0 / 2 added to rows 1 / 3 and the last lane of row 1
// added to rows 2 and 3 (the gfx9 row broadcasts). Lanes whose DPP source is out of range add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_inclusive_scan(float x) {
    x += dpp_or_zero<0x111, 0xf>(x);  // row_shr:1
    x += dpp_or_zero<0x112, 0xf>(x);  // row_shr:2
    x += dpp_or_zero<0x114, 0xf>(x);  // row_shr:4
    x += dpp_or_zero<0x118, 0xf>(x);  // row_shr:8
    x += dpp_or_zero<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_or_zero<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// blockIdx -> (chain, sub-block) so that all sub-blocks of one chain run on
// the same XCD (workgroups are dispatched round-robin over the 8 XCDs, so
// consecutive linear ids land on different XCDs; each XCD has its own L2).
// The grid must hold ceil(chains / 8) * 8 * nsub workgroups.
__device__ __forceinline__ void xcd_split(int L, int nsub, int& chain, int& sub) {
    const int xcd = L & 7, idx = L >> 3;
    chain = (idx / nsub) * 8 + xcd;
    sub = idx % nsub;
}

// 16-byte direct load global -> LDS: lane l's 16 bytes land at dst + 16 l.
__device__ __forceinline__ void load_lds16(const void* src, void* dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

// One v_mfma_f32_16x16x32_bf16: lane (ln, lg) brings A[ln][8 lg + j] and B[8 lg + j][ln], j = 0..7
// (any pairing of the 32 reduction slots works as long as both operands use the same one).
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat8(i16x4 x, i16x4 y) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Rows of KD 16-bit elements in LDS (K, Q, V tiles): 1 KB blocks of whole rows; the 16-byte piece b
// of row r sits at piece b ^ swz(r) of its row (KD = 64 or 128). The row-fragment reads (16 rows,
// one piece) and the transposed reads that build transposed fragments (4 rows x 4 pieces per 16
// lanes) both hit 16 different bank groups. The swizzle repeats every 16 rows, so a tile of 16 more
// rows sits (16 / RPB) KB further on.
template <int KD>
struct RowBlock {
    static constexpr int RB = 2 * KD;          // bytes per row
    static constexpr int RPB = 1024 / RB;      // rows per 1 KB block
    static constexpr int PCS = RB / 16;        // 16-byte pieces per row
    static constexpr int BYTES = 64 * RB;      // one 64-row chunk
    static constexpr int NLOAD = BYTES / 1024; // direct-load instructions per chunk
    __device__ static int swz(int r) {
        return KD == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }
    __device__ static int off(int r, int b) { return (r / RPB) * 1024 + (r % RPB) * RB + ((b ^ swz(r)) * 16); }
};

}  // namespace sf

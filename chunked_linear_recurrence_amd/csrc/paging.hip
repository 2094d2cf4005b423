// Paged state cache around the delta-rule chunk forward (attention-gym "Linear Attention", the
// paged_chunk_gdn entry): sequence n starts from slot state_indices[n] of a float32 or bf16 pool
// (zeros when its has_initial_state entry is 0) and its final state overwrites that slot; a
// non-positive index (or one past the pool) gives zero output rows and leaves the pool alone.
// Three elementwise kernels run around the unchanged chunk path: gather the entry states into a
// float32 [N, H, V, K] buffer, scatter the final states back, zero the rows of null sequences.
// The states are a few MB against the tokens' GB, so the extra passes cost little.
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {
namespace {

template <typename PT> struct PoolIo;
template <> struct PoolIo<float> {
    static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ void store(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
};
template <> struct PoolIo<bf16_t> {
    static __device__ __forceinline__ f32x4 load(const bf16_t* p) {
        return Elem<bf16_t>::unpack(*reinterpret_cast<const i16x4*>(p));
    }
    static __device__ __forceinline__ void store(bf16_t* p, f32x4 x) { *reinterpret_cast<i16x4*>(p) = Elem<bf16_t>::pack(x); }
};

__device__ __forceinline__ bool slot_ok(int slot, int num_slots) { return slot > 0 && slot < num_slots; }

// h0[n] = pool[slot n] (or zeros); one thread per four elements, blockIdx.y = sequence
template <typename PT>
__global__ __launch_bounds__(256) void state_gather_kernel(const PT* __restrict__ pool, long long slot_stride, int num_slots,
                                                           const int32_t* __restrict__ idx, const uint8_t* __restrict__ has_init,
                                                           long block, float* __restrict__ h0) {
    const int n = blockIdx.y;
    const int slot = idx[n];
    const bool load = slot_ok(slot, num_slots) && (has_init == nullptr || has_init[n] != 0);
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; 4 * i < block; i += (long)gridDim.x * blockDim.x) {
        const f32x4 x = load ? PoolIo<PT>::load(pool + (size_t)slot * (size_t)slot_stride + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(h0 + (size_t)n * block + 4 * i) = x;
    }
}

// pool[slot n] = ht[n] for the sequences with a slot
template <typename PT>
__global__ __launch_bounds__(256) void state_scatter_kernel(PT* __restrict__ pool, long long slot_stride, int num_slots,
                                                            const int32_t* __restrict__ idx, long block,
                                                            const float* __restrict__ ht) {
    const int n = blockIdx.y;
    const int slot = idx[n];
    if (!slot_ok(slot, num_slots)) return;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; 4 * i < block; i += (long)gridDim.x * blockDim.x)
        PoolIo<PT>::store(pool + (size_t)slot * (size_t)slot_stride + 4 * i,
                          *reinterpret_cast<const f32x4*>(ht + (size_t)n * block + 4 * i));
}

// zero the output rows of null sequences: blockIdx.y = sequence, rows of H*V elements
template <typename ET>
__global__ __launch_bounds__(256) void null_rows_kernel(const int32_t* __restrict__ idx, int num_slots,
                                                        const int32_t* __restrict__ cu, int T, int HV, ET* __restrict__ out) {
    const int n = blockIdx.y;
    if (slot_ok(idx[n], num_slots)) return;
    const long bos = cu ? (long)cu[n] : (long)n * T, eos = cu ? (long)cu[n + 1] : (long)(n + 1) * T;
    const long total = (eos - bos) * HV;
    ET* o = out + bos * HV;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) o[i] = ET(0);
}

unsigned blocks_for(long vectors) {
    const long b = (vectors + 255) / 256;
    return (unsigned)(b < 1 ? 1 : (b > 256 ? 256 : b));
}

}  // namespace

hipError_t launch_state_gather(bool pool_bf16, const void* pool, long long slot_stride, int num_slots, const int32_t* idx,
                               const uint8_t* has_init, int N, long block, float* h0, hipStream_t s) {
    if (N == 0) return hipSuccess;
    const dim3 grid(blocks_for(block / 4), (unsigned)N);
    timing_begin("state_gather", s);
    if (pool_bf16)
        state_gather_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(pool), slot_stride, num_slots, idx,
                                                         has_init, block, h0);
    else
        state_gather_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(pool), slot_stride, num_slots, idx,
                                                        has_init, block, h0);
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_state_scatter(bool pool_bf16, void* pool, long long slot_stride, int num_slots, const int32_t* idx,
                                int N, long block, const float* ht, hipStream_t s) {
    if (N == 0) return hipSuccess;
    const dim3 grid(blocks_for(block / 4), (unsigned)N);
    timing_begin("state_scatter", s);
    if (pool_bf16)
        state_scatter_kernel<bf16_t><<<grid, 256, 0, s>>>(static_cast<bf16_t*>(pool), slot_stride, num_slots, idx, block, ht);
    else
        state_scatter_kernel<float><<<grid, 256, 0, s>>>(static_cast<float*>(pool), slot_stride, num_slots, idx, block, ht);
    timing_end(s);
    return hipGetLastError();
}

hipError_t launch_null_rows(bool bf16, const int32_t* idx, int num_slots, const int32_t* cu, int N, int T, int HV,
                            void* out, hipStream_t s) {
    if (N == 0) return hipSuccess;
    const dim3 grid(64, (unsigned)N);
    timing_begin("null_rows", s);
    if (bf16)
        null_rows_kernel<bf16_t><<<grid, 256, 0, s>>>(idx, num_slots, cu, T, HV, static_cast<bf16_t*>(out));
    else
        null_rows_kernel<float><<<grid, 256, 0, s>>>(idx, num_slots, cu, T, HV, static_cast<float*>(out));
    timing_end(s);
    return hipGetLastError();
}

}  // namespace sf

// Internal interface between the host entry points (sf_api.hip) and the
// kernel launchers (gdn.hip, gla.hip, scan.hip). Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sf {

constexpr int kGdnChunk = 64;

// Bytes of one per-(chunk, head) factor record of the delta-rule "Pre" stage. float32: the 64x64 solve
// factor T, the 64x64 decay-masked query-key block P (row-major float32) and 256 float coefficients. bf16:
// T diag(beta) as six 1 KB MFMA fragments of its lower-triangular blocks and the 256 coefficients (the bf16
// chain kernels form P themselves).
constexpr size_t kGdnRecordBf16 = 6 * 1024 + 256 * sizeof(float);
__host__ __device__ inline size_t gdn_factor_bytes(int elem_bytes) {
    return elem_bytes == 2 ? kGdnRecordBf16
                           : (size_t)2 * kGdnChunk * kGdnChunk * elem_bytes + 256 * sizeof(float);
}

// Locate chunk `slot`: batch row, first token, length, index of the chunk in
// its sequence. false past the end.
__device__ __forceinline__ bool chunk_coords(int slot, const int2* table, const int32_t* cu, int T,
                                             int nc, int& b, int& t0, int& L, int& ci) {
    if (table) {
        const int2 e = table[slot];
        if (e.x < 0) return false;
        b = 0;
        t0 = cu[e.x] + kGdnChunk * e.y;
        L = min(kGdnChunk, cu[e.x + 1] - t0);
        ci = e.y;
    } else {
        b = slot / nc;
        ci = slot % nc;
        t0 = ci * kGdnChunk;
        L = min(kGdnChunk, T - t0);
    }
    return true;
}
__device__ __forceinline__ bool chunk_coords(int slot, const int2* table, const int32_t* cu, int T,
                                             int nc, int& b, int& t0, int& L) {
    int ci;
    return chunk_coords(slot, table, cu, T, nc, b, t0, L, ci);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace carve-up for the delta-rule path (packed: chunk offsets + table).
struct GdnWorkspace {
    int* chunk_off;      // [N + 1] (packed only)
    int2* table;         // [cap]   (packed only)
    uint8_t* factors;    // [slots, H] records
    size_t bytes;
};

// Number of chunk slots: dense B * ceil(T/64); packed ceil(T/64) + N.
inline long gdn_slots(int B, int T, int N, bool packed) {
    const long nc = (T + kGdnChunk - 1) / kGdnChunk;
    return packed ? nc + N : (long)B * nc;
}

inline GdnWorkspace gdn_workspace_layout(void* base, int elem_bytes, int B, int T, int H, int N,
                                         bool packed) {
    GdnWorkspace w{};
    size_t off = 0;
    uint8_t* p = static_cast<uint8_t*>(base);
    const long slots = gdn_slots(B, T, N, packed);
    if (packed) {
        w.chunk_off = reinterpret_cast<int*>(p ? p + off : nullptr);
        off += align256(sizeof(int) * (size_t)(N + 1));
        w.table = reinterpret_cast<int2*>(p ? p + off : nullptr);
        off += align256(sizeof(int2) * (size_t)slots);
    }
    w.factors = p ? p + off : nullptr;
    off += align256(gdn_factor_bytes(elem_bytes) * (size_t)slots * H);
    w.bytes = off;
    return w;
}

// Workspace of the delta-rule chunk backward: the chunk table of packed inputs, one record per (chunk slot,
// head) (T [64][64], W and Qt [64][K] in the input type in float32-sized regions, 256 float32
// coefficients), every chunk's float32 entry state and the gradient of every chunk's exit state ([slots][H][V][K]
// each).
struct GdnBwdWorkspace {
    int* chunk_off;
    int2* table;
    float* rec;
    float* states;
    float* dstates;
    size_t bytes;
};
inline size_t gdn_bwd_record_floats(int K) {
    return (size_t)kGdnChunk * kGdnChunk + 2 * (size_t)kGdnChunk * K + 256;
}
inline GdnBwdWorkspace gdn_bwd_workspace_layout(void* base, int B, int T, int H, int K, int V, int N, bool packed) {
    GdnBwdWorkspace w{};
    size_t off = 0;
    uint8_t* p = static_cast<uint8_t*>(base);
    const long slots = gdn_slots(B, T, N, packed);
    auto take = [&](size_t bytes) {
        uint8_t* r = p ? p + off : nullptr;
        off += align256(bytes);
        return r;
    };
    if (packed) {
        w.chunk_off = reinterpret_cast<int*>(take(sizeof(int) * (size_t)(N + 1)));
        w.table = reinterpret_cast<int2*>(take(sizeof(int2) * (size_t)slots));
    }
    w.rec = reinterpret_cast<float*>(take(sizeof(float) * gdn_bwd_record_floats(K) * (size_t)slots * H));
    w.states = reinterpret_cast<float*>(take(sizeof(float) * (size_t)slots * H * V * K));
    w.dstates = reinterpret_cast<float*>(take(sizeof(float) * (size_t)slots * H * V * K));
    w.bytes = off;
    return w;
}

// Workspace of the KDA chunk forward: the chunk table of packed inputs and one float32 record per (chunk
// slot, head) (W, U, P, Qg, Kh, Gamma_L; kda_record_floats floats).
struct KdaWorkspace {
    int* chunk_off;
    int2* table;
    float* rec;
    size_t bytes;
};
size_t kda_record_floats(int K, int V);
inline KdaWorkspace kda_workspace_layout(void* base, int B, int T, int H, int K, int V, int N, bool packed) {
    KdaWorkspace w{};
    size_t off = 0;
    uint8_t* p = static_cast<uint8_t*>(base);
    const long slots = gdn_slots(B, T, N, packed);
    if (packed) {
        w.chunk_off = reinterpret_cast<int*>(p ? p + off : nullptr);
        off += align256(sizeof(int) * (size_t)(N + 1));
        w.table = reinterpret_cast<int2*>(p ? p + off : nullptr);
        off += align256(sizeof(int2) * (size_t)slots);
    }
    w.rec = reinterpret_cast<float*>(p ? p + off : nullptr);
    off += align256(sizeof(float) * kda_record_floats(K, V) * (size_t)slots * H);
    w.bytes = off;
    return w;
}

// Raw gate projection read by the delta-rule Pre stage in place of g (the gate transform fused
// into its gate load): g = -exp(A_log[h]) softplus(raw + dt_bias[h]) or, bounded,
// lower_bound sigmoid(exp(A_log[h]) (raw + dt_bias[h])). raw == nullptr: read g as given.
struct GateSrc {
    const void* raw;
    int raw_bf16;
    const float* A_log;
    const float* dt_bias;
    int bounded;
    float lower_bound;
};

// Measurement hook (see sf_timing_enable): brackets one launch with events.
void timing_begin(const char* name, hipStream_t s);
void timing_end(hipStream_t s);

// ---- launchers (return the HIP error of the launch) ----
hipError_t launch_chunk_table(const int32_t* cu, int N, int chunk, long cap, int* chunk_off,
                              int2* table, hipStream_t s);

// mode: 0 = forward (writes out/ht), 1 = summary (writes S_ext into ht, M into Mout).
// stages: 1 = Pre (and the chunk table) into the workspace, 2 = the chain from the workspace's
// records, 3 = both. Pre's records serve both modes.
hipError_t launch_gdn(bool bf16, int mode, const void* q, const void* k, const void* v,
                      const float* g, const float* beta, const float* h0, const int32_t* cu,
                      const GdnWorkspace& ws, int N, int B, int T, int H, int HK, int K, int V,
                      float scale, void* out, float* ht, float* Mout, hipStream_t s, int stages = 3,
                      const GateSrc* gate_src = nullptr);

// Delta-rule chunk backward (gdn_bwd.hip): dq, dk, dv in the input type, dg, dbeta float32 [B, T, H], dh0
// float32 [N, H, V, K] (or null) for upstream gradients dout [B, T, H, V] (input type) and dht (or null:
// zero). Needs HK == H.
hipError_t launch_gdn_bwd(bool bf16, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* h0, const void* dout, const float* dht,
                          const int32_t* cu, const GdnBwdWorkspace& ws, int N, int B, int T, int H, int K,
                          int V, float scale, void* dq, void* dk, void* dv, float* dg, float* dbeta,
                          float* dh0, hipStream_t s);

// KDA chunk forward (kda.hip): q, k, g [B, T, H, K], v and out [B, T, H, V] (g float32), beta [B, T, H].
// (K, V) in {(128, 128), (128, 64), (64, 64)}.
hipError_t launch_kda_chunk(bool bf16, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* h0, const int32_t* cu, const KdaWorkspace& ws, int N,
                            int B, int T, int H, int K, int V, float scale, void* out, float* ht, hipStream_t s);

// Paged state cache around the chunk path (paging.hip). block = H*V*K elements per slot.
hipError_t launch_state_gather(bool pool_bf16, const void* pool, long long slot_stride, int num_slots, const int32_t* idx,
                               const uint8_t* has_init, int N, long block, float* h0, hipStream_t s);
hipError_t launch_state_scatter(bool pool_bf16, void* pool, long long slot_stride, int num_slots, const int32_t* idx,
                                int N, long block, const float* ht, hipStream_t s);
hipError_t launch_null_rows(bool bf16, const int32_t* idx, int num_slots, const int32_t* cu, int N, int T, int HV,
                            void* out, hipStream_t s);

// Gate transform (gates.hip): n elements of raw [rows, H, D] -> float32 decays.
hipError_t launch_gate_transform(bool bf16, bool bounded, const void* raw, const float* A_log, const float* dt_bias,
                                 long n, int H, int D, float lower_bound, float* out, hipStream_t s);

// Token-by-token delta-rule forward (decode.hip): the state from h0 (or zero) to ht, or, when
// pool is non-null, from and back to the slots state_indices name (pool_bf16: its element type).
// per_channel: Kimi Delta Attention, g [B, T, H, K] (one decay per key channel), HK == H.
hipError_t launch_gdn_recurrent(bool bf16, bool pool_bf16, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, const float* h0, float* ht, void* pool,
                                long long slot_stride, int num_slots, const int32_t* state_indices,
                                const uint8_t* has_init, const int32_t* cu, int N, int T, int H, int HK, int K,
                                int V, float scale, void* out, hipStream_t s, bool per_channel = false);

// One-token paged delta-rule decode (decode.hip). pool_bf16: the pool's element type.
hipError_t launch_gdn_decode(bool bf16, bool pool_bf16, const void* qkv, const void* raw_gate,
                             const void* raw_beta, const float* A_log, const float* dt_bias, void* pool,
                             long long slot_stride, int num_slots, const int32_t* state_indices,
                             const uint8_t* has_init, int B, int H, int HK, int K, int V, float scale,
                             void* out, hipStream_t s, bool per_channel = false, int bounded = 0,
                             float lower_bound = 0.f);

// Compute units of the current device, and whether a bf16 delta-rule forward chain over `chains`
// (sequence, head) pairs of V state rows runs per 16-row slice (else per head).
int device_cus();
bool gdn_chain_per_slice(long chains, int V);

hipError_t launch_gla(bool bf16, int mode, const void* q, const void* k, const void* v,
                      const float* g, const float* h0, const int32_t* cu, int N, int B, int T,
                      int H, int HK, int K, int V, int chunk, float scale, void* out, float* ht,
                      float* a_out, hipStream_t s);

hipError_t launch_scan(int kind, const float* M, const float* S_ext, const float* h0, int B,
                       int n_seg, int H, int K, int V, float* S_in, float* S_final, hipStream_t s);

}  // namespace sf

// Host entry points of the C ABI declared in include/sf.h: argument
// validation, workspace carve-up and kernel dispatch. No allocation, no
// synchronisation on the enqueue path.
#include "../../include/sf.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "sf_internal.h"

namespace {

thread_local char g_err[512] = "";

sf_status fail(sf_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

sf_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return SF_OK;
    return fail(SF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr long kMaxElems = 0x7fffffffL;

bool fits(long a) { return a >= 0 && a <= kMaxElems; }

int elem_bytes(sf_dtype dt) { return dt == SF_BF16 ? 2 : 4; }

// Common shape checks for token-major inputs.
// The chunk kernels move q, k, v and the output rows in 16-byte pieces.
sf_status check_rows16(std::initializer_list<const void*> ps, const char* names) {
    for (const void* p : ps)
        if (p && reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(SF_ERR_INVALID, "%s must be 16-byte aligned (moved in 16-byte pieces)", names);
    return SF_OK;
}

sf_status check_tokens(sf_dtype dt, int B, int T, int H, int HK, int K, int V, int N,
                       bool packed) {
    if (dt != SF_F32 && dt != SF_BF16) return fail(SF_ERR_INVALID, "dtype must be SF_F32 or SF_BF16");
    if (B < 0 || T < 0 || H <= 0 || HK <= 0 || K <= 0 || V <= 0 || N < 0)
        return fail(SF_ERR_INVALID, "sizes must be positive (B=%d T=%d H=%d HK=%d K=%d V=%d N=%d)", B, T, H,
                    HK, K, V, N);
    if (H % HK != 0) return fail(SF_ERR_INVALID, "HK=%d must divide H=%d", HK, H);
    if (packed && B != 1) return fail(SF_ERR_INVALID, "cu_seqlens needs batch-one inputs (B=%d)", B);
    if (!packed && N != B) return fail(SF_ERR_INVALID, "without cu_seqlens N (%d) must equal B (%d)", N, B);
    if (!fits((long)B * T * HK * K) || !fits((long)B * T * H * V) || !fits((long)N * H * V * K) ||
        !fits((long)B * T * H))
        return fail(SF_ERR_UNSUPPORTED, "a tensor has 2^31 or more elements (int64 offsets are not supported)");
    return SF_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// timing hook
// ---------------------------------------------------------------------------
namespace sf {
namespace {
struct TimingRec {
    const char* name;
    int pair;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<hipEvent_t> g_ev;  // 2 * pairs
std::vector<TimingRec> g_recs;
int g_next = 0;
const char* g_pending = nullptr;
}  // namespace

void timing_begin(const char* name, hipStream_t s) {
    if (!g_timing) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    g_pending = nullptr;
    if (2 * (g_next + 1) > (int)g_ev.size()) return;
    if (hipEventRecord(g_ev[2 * g_next], s) != hipSuccess) return;
    g_pending = name;
}

void timing_end(hipStream_t s) {
    if (!g_timing) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!g_pending) return;
    if (hipEventRecord(g_ev[2 * g_next + 1], s) == hipSuccess) g_recs.push_back({g_pending, g_next++});
    g_pending = nullptr;
}
}  // namespace sf

extern "C" {

const char* sf_version(void) { return "sf 0.1.0 gfx950"; }

const char* sf_last_error(void) { return g_err; }

sf_status sf_timing_enable(int max_pairs) {
    std::lock_guard<std::mutex> lk(sf::g_tmu);
    for (hipEvent_t e : sf::g_ev) (void)hipEventDestroy(e);
    sf::g_ev.clear();
    sf::g_recs.clear();
    sf::g_next = 0;
    sf::g_timing = false;
    if (max_pairs <= 0) return SF_OK;
    sf::g_ev.resize(2 * (size_t)max_pairs);
    for (auto& e : sf::g_ev) {
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return hip_status(err, "hipEventCreate");
    }
    sf::g_timing = true;
    return SF_OK;
}

int sf_timing_collect(const char** names, double* total_ms, int* launches, int max_kernels) {
    std::lock_guard<std::mutex> lk(sf::g_tmu);
    int nk = 0;
    for (const auto& r : sf::g_recs) {
        if (hipEventSynchronize(sf::g_ev[2 * r.pair + 1]) != hipSuccess) return -1;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, sf::g_ev[2 * r.pair], sf::g_ev[2 * r.pair + 1]) != hipSuccess) return -1;
        int i = 0;
        while (i < nk && strcmp(names[i], r.name) != 0) ++i;
        if (i == nk) {
            if (nk == max_kernels) continue;
            names[nk] = r.name;
            total_ms[nk] = 0.0;
            launches[nk] = 0;
            ++nk;
        }
        total_ms[i] += ms;
        launches[i] += 1;
    }
    sf::g_recs.clear();
    sf::g_next = 0;
    return nk;
}

sf_status sf_check_cu_seqlens(const int32_t* cu, int N, int T) {
    if (N < 0 || T < 0) return fail(SF_ERR_INVALID, "N and T must be nonnegative (N=%d T=%d)", N, T);
    if (!cu) return fail(SF_ERR_INVALID, "cu_seqlens is NULL");
    if (cu[0] != 0) return fail(SF_ERR_INVALID, "cu_seqlens[0] is %d, must be 0", (int)cu[0]);
    for (int n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n])
            return fail(SF_ERR_INVALID, "cu_seqlens decreases at %d: %d -> %d", n, (int)cu[n], (int)cu[n + 1]);
    if (cu[N] > T) return fail(SF_ERR_INVALID, "cu_seqlens[%d] = %d is past T = %d", N, (int)cu[N], T);
    return SF_OK;
}

sf_status sf_check_state_indices(const int32_t* idx, int N, int num_slots) {
    if (N < 0 || num_slots < 0) return fail(SF_ERR_INVALID, "N and num_slots must be nonnegative");
    if (N > 0 && !idx) return fail(SF_ERR_INVALID, "state_indices is NULL");
    std::vector<int> owner((size_t)num_slots, -1);
    for (int n = 0; n < N; ++n) {
        const int s = idx[n];
        if (s <= 0) continue;
        if (s >= num_slots) return fail(SF_ERR_INVALID, "state_indices[%d] = %d is past num_slots = %d", n, s, num_slots);
        if (owner[(size_t)s] >= 0)
            return fail(SF_ERR_INVALID, "state_indices[%d] and [%d] both name slot %d (they would race)", owner[(size_t)s], n, s);
        owner[(size_t)s] = n;
    }
    return SF_OK;
}

size_t sf_gdn_chunk_fwd_workspace(sf_dtype dt, int B, int T, int H, int K, int V, int N, int packed) {
    (void)K;
    (void)V;
    if ((dt != SF_F32 && dt != SF_BF16) || B < 0 || T < 0 || H <= 0 || N < 0) return 0;
    return sf::gdn_workspace_layout(nullptr, elem_bytes(dt), B, T, H, N, packed != 0).bytes;
}

sf_status sf_gdn_chunk_fwd(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* h0, const int32_t* cu_seqlens, int N, int B,
                           int T, int H, int HK, int K, int V, float scale, void* out, float* ht,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    sf_status st = check_tokens(dt, B, T, H, HK, K, V, N, packed);
    if (st != SF_OK) return st;
    if ((st = check_rows16({q, k, v, out}, "q, k, v and out")) != SF_OK) return st;
    if (!q || !k || !v || !g || !beta || !out) return fail(SF_ERR_INVALID, "q, k, v, g, beta and out must not be NULL");
    if (K != V || (K != 64 && K != 128))
        return fail(SF_ERR_UNSUPPORTED, "delta-rule kernels are built for K == V in {64, 128} (K=%d V=%d)", K, V);
    const sf::GdnWorkspace need = sf::gdn_workspace_layout(nullptr, elem_bytes(dt), B, T, H, N, packed);
    if (!workspace || workspace_bytes < need.bytes)
        return fail(SF_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                    need.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(SF_ERR_INVALID, "workspace must be 256-byte aligned");
    const sf::GdnWorkspace ws = sf::gdn_workspace_layout(workspace, elem_bytes(dt), B, T, H, N, packed);
    hipError_t e = sf::launch_gdn(dt == SF_BF16, 0, q, k, v, g, beta, h0, cu_seqlens, ws, N, B, T, H, HK, K, V,
                                  scale, out, ht, nullptr, static_cast<hipStream_t>(stream));
    return hip_status(e, "sf_gdn_chunk_fwd launch");
}

// ---------------------------------------------------------------------------
// KDA chunk forward
// ---------------------------------------------------------------------------
size_t sf_kda_chunk_fwd_workspace(sf_dtype dt, int B, int T, int H, int K, int V, int N, int packed) {
    if ((dt != SF_F32 && dt != SF_BF16) || B < 0 || T < 0 || H <= 0 || N < 0) return 0;
    if (!((K == 128 && (V == 128 || V == 64)) || (K == 64 && V == 64))) return 0;
    return sf::kda_workspace_layout(nullptr, B, T, H, K, V, N, packed != 0).bytes;
}

sf_status sf_kda_chunk_fwd(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* h0, const int32_t* cu_seqlens, int N, int B, int T,
                           int H, int K, int V, float scale, void* out, float* ht, void* workspace,
                           size_t workspace_bytes, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    sf_status st = check_tokens(dt, B, T, H, H, K, V, N, packed);
    if (st != SF_OK) return st;
    if ((st = check_rows16({q, k, v, out}, "q, k, v and out")) != SF_OK) return st;
    if (!q || !k || !v || !g || !beta || !out) return fail(SF_ERR_INVALID, "q, k, v, g, beta and out must not be NULL");
    if (!((K == 128 && (V == 128 || V == 64)) || (K == 64 && V == 64)))
        return fail(SF_ERR_UNSUPPORTED, "the KDA chunk forward is built for (K, V) in {(128, 128), (128, 64), (64, 64)} "
                    "(K=%d V=%d)", K, V);
    if (!fits((long)B * T * H * K)) return fail(SF_ERR_UNSUPPORTED, "the gate has 2^31 or more elements");
    if (H > 65535) return fail(SF_ERR_UNSUPPORTED, "H=%d is past the 65535 heads of a launch", H);
    const sf::KdaWorkspace need = sf::kda_workspace_layout(nullptr, B, T, H, K, V, N, packed);
    if (!workspace || workspace_bytes < need.bytes)
        return fail(SF_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                    need.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(SF_ERR_INVALID, "workspace must be 256-byte aligned");
    const sf::KdaWorkspace ws = sf::kda_workspace_layout(workspace, B, T, H, K, V, N, packed);
    hipError_t e = sf::launch_kda_chunk(dt == SF_BF16, q, k, v, g, beta, h0, cu_seqlens, ws, N, B, T, H, K, V, scale,
                                        out, ht, static_cast<hipStream_t>(stream));
    return hip_status(e, "sf_kda_chunk_fwd launch");
}

// ---------------------------------------------------------------------------
// Chunk backward
// ---------------------------------------------------------------------------
size_t sf_gdn_chunk_bwd_workspace(sf_dtype dt, int B, int T, int H, int K, int V, int N, int packed) {
    if ((dt != SF_F32 && dt != SF_BF16) || B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0 || N < 0) return 0;
    return sf::gdn_bwd_workspace_layout(nullptr, B, T, H, K, V, N, packed != 0).bytes;
}

sf_status sf_gdn_chunk_bwd(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* h0, const void* dout, const float* dht,
                           const int32_t* cu_seqlens, int N, int B, int T, int H, int HK, int K, int V,
                           float scale, void* dq, void* dk, void* dv, float* dg, float* dbeta, float* dh0,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    sf_status st = check_tokens(dt, B, T, H, HK, K, V, N, packed);
    if (st != SF_OK) return st;
    if (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta)
        return fail(SF_ERR_INVALID, "q, k, v, g, beta, dout, dq, dk, dv, dg and dbeta must not be NULL");
    if (HK != H) return fail(SF_ERR_UNSUPPORTED, "the chunk backward needs one q/k head per value head (HK=%d H=%d)", HK, H);
    if ((K != 64 && K != 128) || (V != 64 && V != 128))
        return fail(SF_ERR_UNSUPPORTED, "the chunk backward is built for K, V in {64, 128} (K=%d V=%d)", K, V);
    if (H > 65535) return fail(SF_ERR_UNSUPPORTED, "H=%d is past the 65535 heads of a launch", H);
    for (const void* p : {q, k, v, dout, static_cast<const void*>(dq), static_cast<const void*>(dk),
                          static_cast<const void*>(dv)})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
            return fail(SF_ERR_INVALID, "q, k, v, dout, dq, dk and dv must be 16-byte aligned (read and written in 16-byte pieces)");
    const sf::GdnBwdWorkspace need = sf::gdn_bwd_workspace_layout(nullptr, B, T, H, K, V, N, packed);
    if (!workspace || workspace_bytes < need.bytes)
        return fail(SF_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                    need.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(SF_ERR_INVALID, "workspace must be 256-byte aligned");
    const sf::GdnBwdWorkspace ws = sf::gdn_bwd_workspace_layout(workspace, B, T, H, K, V, N, packed);
    hipError_t e = sf::launch_gdn_bwd(dt == SF_BF16, q, k, v, g, beta, h0, dout, dht, cu_seqlens, ws, N, B, T, H, K, V,
                                      scale, dq, dk, dv, dg, dbeta, dh0, static_cast<hipStream_t>(stream));
    return hip_status(e, "sf_gdn_chunk_bwd launch");
}

// ---------------------------------------------------------------------------
// The chunk forward with its workspace in a static device array, for callers that cannot allocate.
// ---------------------------------------------------------------------------
namespace {
// Every GPU the library runs on holds its own copy of this array (module globals are per device)
// until the process ends. Host code never uses its name as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sf_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(SF_ERR_UNSUPPORTED, "device ordinal %d is past %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(SF_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SF_OK;
}
}  // namespace

size_t sf_static_scratch_bytes(void) { return kScratchBytes; }

sf_status sf_gdn_chunk_fwd_noalloc(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* h0, const int32_t* cu_seqlens, int N, int B,
                                   int T, int H, int HK, int K, int V, float scale, void* out, float* ht,
                                   void* stream) {
    const bool packed = cu_seqlens != nullptr;
    sf_status st = check_tokens(dt, B, T, H, HK, K, V, N, packed);
    if (st != SF_OK) return st;
    if ((st = check_rows16({q, k, v, out}, "q, k, v and out")) != SF_OK) return st;
    if (!q || !k || !v || !g || !beta || !out) return fail(SF_ERR_INVALID, "q, k, v, g, beta and out must not be NULL");
    if (K != V || (K != 64 && K != 128))
        return fail(SF_ERR_UNSUPPORTED, "delta-rule kernels are built for K == V in {64, 128} (K=%d V=%d)", K, V);
    const sf::GdnWorkspace need = sf::gdn_workspace_layout(nullptr, elem_bytes(dt), B, T, H, N, packed);
    if (need.bytes > kScratchBytes)
        return fail(SF_ERR_WORKSPACE, "these sizes need %zu bytes of scratch, more than the static %zu", need.bytes,
                    kScratchBytes);
    void* base = nullptr;
    if ((st = scratch_for_current_device(&base)) != SF_OK) return st;
    // nothing in the scratch has to start at zero: every byte a kernel reads was written earlier in this call
    const sf::GdnWorkspace ws = sf::gdn_workspace_layout(base, elem_bytes(dt), B, T, H, N, packed);
    hipError_t e = sf::launch_gdn(dt == SF_BF16, 0, q, k, v, g, beta, h0, cu_seqlens, ws, N, B, T, H, HK, K, V,
                                  scale, out, ht, nullptr, static_cast<hipStream_t>(stream));
    return hip_status(e, "sf_gdn_chunk_fwd_noalloc launch");
}

sf_status sf_gdn_chunk_fwd_raw_gate(sf_dtype dt, const void* q, const void* k, const void* v, const void* raw_gate,
                                    const float* A_log, const float* dt_bias, sf_gate_kind kind, float lower_bound,
                                    const float* beta, const float* h0, const int32_t* cu_seqlens, int N, int B, int T,
                                    int H, int HK, int K, int V, float scale, void* out, float* ht, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    sf_status st = check_tokens(dt, B, T, H, HK, K, V, N, packed);
    if (st != SF_OK) return st;
    if ((st = check_rows16({q, k, v, out}, "q, k, v and out")) != SF_OK) return st;
    if (!q || !k || !v || !raw_gate || !A_log || !dt_bias || !beta || !out)
        return fail(SF_ERR_INVALID, "q, k, v, raw_gate, A_log, dt_bias, beta and out must not be NULL");
    if (kind != SF_GATE_SOFTPLUS && kind != SF_GATE_BOUNDED)
        return fail(SF_ERR_INVALID, "kind must be SF_GATE_SOFTPLUS or SF_GATE_BOUNDED");
    if (kind == SF_GATE_BOUNDED && !(lower_bound <= 0.f && lower_bound > -3.0e38f))
        return fail(SF_ERR_INVALID, "the bounded kind needs a finite lower_bound <= 0 (got %g)", (double)lower_bound);
    if (K != V || (K != 64 && K != 128))
        return fail(SF_ERR_UNSUPPORTED, "delta-rule kernels are built for K == V in {64, 128} (K=%d V=%d)", K, V);
    const sf::GdnWorkspace need = sf::gdn_workspace_layout(nullptr, elem_bytes(dt), B, T, H, N, packed);
    if (!workspace || workspace_bytes < need.bytes)
        return fail(SF_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                    need.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(SF_ERR_INVALID, "workspace must be 256-byte aligned");
    const sf::GdnWorkspace ws = sf::gdn_workspace_layout(workspace, elem_bytes(dt), B, T, H, N, packed);
    const sf::GateSrc gs{raw_gate, dt == SF_BF16 ? 1 : 0, A_log, dt_bias, kind == SF_GATE_BOUNDED ? 1 : 0, lower_bound};
    hipError_t e = sf::launch_gdn(dt == SF_BF16, 0, q, k, v, nullptr, beta, h0, cu_seqlens, ws, N, B, T, H, HK, K, V,
                                  scale, out, ht, nullptr, static_cast<hipStream_t>(stream), 3, &gs);
    return hip_status(e, "sf_gdn_chunk_fwd_raw_gate launch");
}

sf_status sf_gla_chunk_fwd(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                           const float* h0, const int32_t* cu_seqlens, int N, int B, int T, int H, int HK,
                           int K, int V, int chunk, float scale, void* out, float* ht, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    sf_status st = check_tokens(dt, B, T, H, HK, K, V, N, packed);
    if (st != SF_OK) return st;
    if ((st = check_rows16({q, k, v, out}, "q, k, v and out")) != SF_OK) return st;
    if (!q || !k || !v || !g || !out) return fail(SF_ERR_INVALID, "q, k, v, g and out must not be NULL");
    if (chunk != 64 && chunk != 128) return fail(SF_ERR_UNSUPPORTED, "chunk must be 64 or 128 (got %d)", chunk);
    if (dt == SF_F32 && chunk != 64) return fail(SF_ERR_UNSUPPORTED, "float32 inputs use chunk 64");
    if ((K != 64 && K != 128) || (V != 64 && V != 128))
        return fail(SF_ERR_UNSUPPORTED, "scalar-gate kernels are built for K, V in {64, 128} (K=%d V=%d)", K, V);
    hipError_t e = sf::launch_gla(dt == SF_BF16, 0, q, k, v, g, h0, cu_seqlens, N, B, T, H, HK, K, V, chunk, scale,
                                  out, ht, nullptr, static_cast<hipStream_t>(stream));
    return hip_status(e, "sf_gla_chunk_fwd launch");
}

size_t sf_segment_summary_workspace(sf_kind kind, sf_dtype dt, int n_rows, int L_seg, int H, int K, int V,
                                    int chunk) {
    (void)K;
    (void)V;
    (void)chunk;
    if (kind == SF_KIND_GLA) return 0;
    if (kind != SF_KIND_GDN || (dt != SF_F32 && dt != SF_BF16) || n_rows < 0 || L_seg < 0 || H <= 0) return 0;
    return sf::gdn_workspace_layout(nullptr, elem_bytes(dt), n_rows, L_seg, H, n_rows, false).bytes;
}

sf_status sf_segment_summary(sf_kind kind, sf_dtype dt, const void* k, const void* v, const float* g,
                             const float* beta, int n_rows, int L_seg, int H, int HK, int K, int V, int chunk,
                             float* M, float* S_ext, void* workspace, size_t workspace_bytes, void* stream) {
    sf_status st = check_tokens(dt, n_rows, L_seg, H, HK, K, V, n_rows, false);
    if (st != SF_OK) return st;
    if ((st = check_rows16({k, v}, "k and v")) != SF_OK) return st;
    if (!k || !v || !g || !M || !S_ext) return fail(SF_ERR_INVALID, "k, v, g, M and S_ext must not be NULL");
    if (!fits((long)n_rows * H * K * K)) return fail(SF_ERR_UNSUPPORTED, "M has 2^31 or more elements");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind == SF_KIND_GDN) {
        if (!beta) return fail(SF_ERR_INVALID, "beta must not be NULL for SF_KIND_GDN");
        if (chunk != 64) return fail(SF_ERR_UNSUPPORTED, "delta-rule chunk is 64 (got %d)", chunk);
        if (K != V || (K != 64 && K != 128))
            return fail(SF_ERR_UNSUPPORTED, "delta-rule kernels are built for K == V in {64, 128} (K=%d V=%d)", K, V);
        const sf::GdnWorkspace need = sf::gdn_workspace_layout(nullptr, elem_bytes(dt), n_rows, L_seg, H, n_rows, false);
        if (!workspace || workspace_bytes < need.bytes)
            return fail(SF_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                        need.bytes);
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(SF_ERR_INVALID, "workspace must be 256-byte aligned");
        const sf::GdnWorkspace ws = sf::gdn_workspace_layout(workspace, elem_bytes(dt), n_rows, L_seg, H, n_rows, false);
        hipError_t e = sf::launch_gdn(dt == SF_BF16, 1, nullptr, k, v, g, beta, nullptr, nullptr, ws, n_rows, n_rows,
                                      L_seg, H, HK, K, V, 1.f, nullptr, S_ext, M, s);
        return hip_status(e, "sf_segment_summary launch");
    }
    if (kind == SF_KIND_GLA) {
        if (chunk != 64 && chunk != 128) return fail(SF_ERR_UNSUPPORTED, "chunk must be 64 or 128 (got %d)", chunk);
        if (dt == SF_F32 && chunk != 64) return fail(SF_ERR_UNSUPPORTED, "float32 inputs use chunk 64");
        if ((K != 64 && K != 128) || (V != 64 && V != 128))
            return fail(SF_ERR_UNSUPPORTED, "scalar-gate kernels are built for K, V in {64, 128} (K=%d V=%d)", K, V);
        hipError_t e = sf::launch_gla(dt == SF_BF16, 1, nullptr, k, v, g, nullptr, nullptr, n_rows, n_rows, L_seg, H,
                                      HK, K, V, chunk, 1.f, nullptr, S_ext, M, s);
        return hip_status(e, "sf_segment_summary launch");
    }
    return fail(SF_ERR_INVALID, "kind must be SF_KIND_GDN or SF_KIND_GLA");
}

namespace {
// Segmented delta-rule workspace: the per-segment Pre records, then M, S_ext and the entry states.
struct SegWorkspace {
    sf::GdnWorkspace pre;
    float *M, *S_ext, *S_in;
    size_t bytes;
};
SegWorkspace seg_layout(void* base, int eb, int n_rows, int L_seg, int H, int K, int V) {
    SegWorkspace w{};
    w.pre = sf::gdn_workspace_layout(base, eb, n_rows, L_seg, H, n_rows, false);
    size_t off = w.pre.bytes;
    uint8_t* p = static_cast<uint8_t*>(base);
    auto take = [&](size_t n) {
        float* r = reinterpret_cast<float*>(p ? p + off : nullptr);
        off += sf::align256(n * sizeof(float));
        return r;
    };
    w.M = take((size_t)n_rows * H * K * K);
    w.S_ext = take((size_t)n_rows * H * V * K);
    w.S_in = take((size_t)n_rows * H * V * K);
    w.bytes = off;
    return w;
}
}  // namespace

size_t sf_gdn_segmented_fwd_workspace(sf_dtype dt, int B, int n_seg, int T, int H, int K, int V) {
    if ((dt != SF_F32 && dt != SF_BF16) || B < 0 || n_seg <= 0 || T < 0 || T % n_seg || H <= 0 || K <= 0 || V <= 0)
        return 0;
    return seg_layout(nullptr, elem_bytes(dt), B * n_seg, T / n_seg, H, K, V).bytes;
}

sf_status sf_gdn_segmented_fwd(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* h0, int B, int n_seg, int T, int H, int HK,
                               int K, int V, float scale, void* out, float* ht, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (n_seg <= 0 || T % (n_seg > 0 ? n_seg : 1) != 0)
        return fail(SF_ERR_INVALID, "T=%d must be a positive multiple of n_seg=%d", T, n_seg);
    const int L_seg = T / n_seg, n_rows = B * n_seg;
    if (L_seg % sf::kGdnChunk != 0)
        return fail(SF_ERR_INVALID, "the segment length %d must be a multiple of the chunk (%d)", L_seg, sf::kGdnChunk);
    sf_status st = check_tokens(dt, n_rows, L_seg, H, HK, K, V, n_rows, false);
    if (st != SF_OK) return st;
    if ((st = check_rows16({q, k, v, out}, "q, k, v and out")) != SF_OK) return st;
    if (!q || !k || !v || !g || !beta || !out) return fail(SF_ERR_INVALID, "q, k, v, g, beta and out must not be NULL");
    if (K != V || (K != 64 && K != 128))
        return fail(SF_ERR_UNSUPPORTED, "delta-rule kernels are built for K == V in {64, 128} (K=%d V=%d)", K, V);
    if (!fits((long)n_rows * H * K * K)) return fail(SF_ERR_UNSUPPORTED, "M has 2^31 or more elements");
    const SegWorkspace need = seg_layout(nullptr, elem_bytes(dt), n_rows, L_seg, H, K, V);
    if (!workspace || workspace_bytes < need.bytes)
        return fail(SF_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                    need.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(SF_ERR_INVALID, "workspace must be 256-byte aligned");
    const SegWorkspace ws = seg_layout(workspace, elem_bytes(dt), n_rows, L_seg, H, K, V);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = dt == SF_BF16;
    // Pre once on the segment view (its records serve both passes), then the summary pass, the exclusive
    // scan and the forward pass from the true entry states
    hipError_t e = sf::launch_gdn(bf, 0, q, k, v, g, beta, nullptr, nullptr, ws.pre, n_rows, n_rows, L_seg, H, HK, K, V,
                                  scale, nullptr, nullptr, nullptr, s, 1);
    if (e == hipSuccess)
        e = sf::launch_gdn(bf, 1, nullptr, k, v, g, beta, nullptr, nullptr, ws.pre, n_rows, n_rows, L_seg, H, HK, K, V,
                           1.f, nullptr, ws.S_ext, ws.M, s, 2);
    if (e == hipSuccess) e = sf::launch_scan(0, ws.M, ws.S_ext, h0, B, n_seg, H, K, V, ws.S_in, ht, s);
    if (e == hipSuccess)
        e = sf::launch_gdn(bf, 0, q, k, v, g, beta, ws.S_in, nullptr, ws.pre, n_rows, n_rows, L_seg, H, HK, K, V,
                           scale, out, nullptr, nullptr, s, 2);
    return hip_status(e, "sf_gdn_segmented_fwd launch");
}

sf_status sf_state_scan(sf_kind kind, const float* M, const float* S_ext, const float* h0, int B, int n_seg,
                        int H, int K, int V, float* S_in, float* S_final, void* stream) {
    if (kind != SF_KIND_GDN && kind != SF_KIND_GLA) return fail(SF_ERR_INVALID, "kind must be SF_KIND_GDN or SF_KIND_GLA");
    if (B < 0 || n_seg < 0 || H <= 0 || K <= 0 || V <= 0) return fail(SF_ERR_INVALID, "sizes must be positive");
    if (!M || !S_ext || !S_in) return fail(SF_ERR_INVALID, "M, S_ext and S_in must not be NULL");
    if (!fits((long)B * n_seg * H * V * K) || !fits((long)B * n_seg * H * K * K))
        return fail(SF_ERR_UNSUPPORTED, "a tensor has 2^31 or more elements");
    if (kind == SF_KIND_GDN) {
        if ((K != 64 && K != 128) || V % 16 != 0)
            return fail(SF_ERR_UNSUPPORTED, "delta-rule scan is built for K in {64, 128} and V a multiple of 16 (K=%d V=%d)",
                        K, V);
    } else if ((V * K) % 4 != 0) {
        return fail(SF_ERR_UNSUPPORTED, "V * K must be a multiple of 4");
    }
    hipError_t e = sf::launch_scan(kind == SF_KIND_GDN ? 0 : 1, M, S_ext, h0, B, n_seg, H, K, V, S_in, S_final,
                                   static_cast<hipStream_t>(stream));
    return hip_status(e, "sf_state_scan launch");
}

namespace {
// paged chunk forward: the chunk path's workspace, then float32 entry and exit states
struct PagedWorkspace {
    sf::GdnWorkspace chunk;
    float *h0, *ht;
    size_t bytes;
};
PagedWorkspace paged_layout(void* base, int eb, int B, int T, int H, int K, int V, int N, bool packed) {
    PagedWorkspace w{};
    w.chunk = sf::gdn_workspace_layout(base, eb, B, T, H, N, packed);
    size_t off = w.chunk.bytes;
    uint8_t* p = static_cast<uint8_t*>(base);
    const size_t st = sf::align256(sizeof(float) * (size_t)N * H * V * K);
    w.h0 = reinterpret_cast<float*>(p ? p + off : nullptr);
    off += st;
    w.ht = reinterpret_cast<float*>(p ? p + off : nullptr);
    off += st;
    w.bytes = off;
    return w;
}
}  // namespace

size_t sf_paged_gdn_chunk_fwd_workspace(sf_dtype dt, int B, int T, int H, int K, int V, int N, int packed) {
    if ((dt != SF_F32 && dt != SF_BF16) || B < 0 || T < 0 || H <= 0 || K <= 0 || V <= 0 || N < 0) return 0;
    return paged_layout(nullptr, elem_bytes(dt), B, T, H, K, V, N, packed != 0).bytes;
}

sf_status sf_paged_gdn_chunk_fwd(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const int32_t* cu_seqlens, int N, int B, int T, int H, int HK, int K,
                                 int V, float scale, void* out, void* state_pool, sf_dtype pool_dt, int num_slots,
                                 long long slot_stride, const int32_t* state_indices, const uint8_t* has_initial_state,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    sf_status st = check_tokens(dt, B, T, H, HK, K, V, N, packed);
    if (st != SF_OK) return st;
    if ((st = check_rows16({q, k, v, out}, "q, k, v and out")) != SF_OK) return st;
    if (!q || !k || !v || !g || !beta || !out) return fail(SF_ERR_INVALID, "q, k, v, g, beta and out must not be NULL");
    if (K != V || (K != 64 && K != 128))
        return fail(SF_ERR_UNSUPPORTED, "delta-rule kernels are built for K == V in {64, 128} (K=%d V=%d)", K, V);
    if (pool_dt != SF_F32 && pool_dt != SF_BF16) return fail(SF_ERR_INVALID, "pool dtype must be SF_F32 or SF_BF16");
    const long long blk = (long long)H * V * K;
    if (num_slots < 0 || slot_stride < blk || slot_stride % 4 != 0)
        return fail(SF_ERR_INVALID, "slot_stride %lld must be a multiple of 4 and at least H*V*K = %lld", slot_stride, blk);
    if (!state_pool || !state_indices) return fail(SF_ERR_INVALID, "state_pool and state_indices must not be NULL");
    if (reinterpret_cast<uintptr_t>(state_pool) % 16 != 0) return fail(SF_ERR_INVALID, "state_pool must be 16-byte aligned");
    const PagedWorkspace need = paged_layout(nullptr, elem_bytes(dt), B, T, H, K, V, N, packed);
    if (!workspace || workspace_bytes < need.bytes)
        return fail(SF_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need.bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return fail(SF_ERR_INVALID, "workspace must be 256-byte aligned");
    const PagedWorkspace ws = paged_layout(workspace, elem_bytes(dt), B, T, H, K, V, N, packed);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool pb = pool_dt == SF_BF16;
    hipError_t e = sf::launch_state_gather(pb, state_pool, slot_stride, num_slots, state_indices, has_initial_state, N,
                                           (long)blk, ws.h0, s);
    if (e == hipSuccess)
        e = sf::launch_gdn(dt == SF_BF16, 0, q, k, v, g, beta, ws.h0, cu_seqlens, ws.chunk, N, B, T, H, HK, K, V, scale,
                           out, ws.ht, nullptr, s);
    if (e == hipSuccess) e = sf::launch_state_scatter(pb, state_pool, slot_stride, num_slots, state_indices, N, (long)blk, ws.ht, s);
    if (e == hipSuccess) e = sf::launch_null_rows(dt == SF_BF16, state_indices, num_slots, cu_seqlens, N, T, H * V, out, s);
    return hip_status(e, "sf_paged_gdn_chunk_fwd launch");
}

sf_status sf_gate_transform(sf_dtype dt, const void* raw, const float* A_log, const float* dt_bias, long long rows,
                            int H, int D, sf_gate_kind kind, float lower_bound, float* out, void* stream) {
    if (dt != SF_F32 && dt != SF_BF16) return fail(SF_ERR_INVALID, "dtype must be SF_F32 or SF_BF16");
    if (kind != SF_GATE_SOFTPLUS && kind != SF_GATE_BOUNDED)
        return fail(SF_ERR_INVALID, "kind must be SF_GATE_SOFTPLUS or SF_GATE_BOUNDED");
    if (rows < 0 || H <= 0 || D <= 0) return fail(SF_ERR_INVALID, "sizes must be positive (rows=%lld H=%d D=%d)", rows, H, D);
    if (kind == SF_GATE_BOUNDED && !(lower_bound <= 0.f && lower_bound > -3.0e38f))
        return fail(SF_ERR_INVALID, "the bounded kind needs a finite lower_bound <= 0 (got %g)", (double)lower_bound);
    if ((long long)H * D > kMaxElems || rows > (1LL << 40) / ((long long)H * D))
        return fail(SF_ERR_UNSUPPORTED, "too many elements");
    if (rows == 0) return SF_OK;
    if (!raw || !A_log || !dt_bias || !out) return fail(SF_ERR_INVALID, "raw, A_log, dt_bias and out must not be NULL");
    if (reinterpret_cast<uintptr_t>(raw) % (dt == SF_BF16 ? 8 : 16) != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return fail(SF_ERR_INVALID, "raw must be %d-byte and out 16-byte aligned", dt == SF_BF16 ? 8 : 16);
    hipError_t e = sf::launch_gate_transform(dt == SF_BF16, kind == SF_GATE_BOUNDED, raw, A_log, dt_bias,
                                             (long)(rows * H * D), H, D, lower_bound, out,
                                             static_cast<hipStream_t>(stream));
    return hip_status(e, "sf_gate_transform launch");
}

namespace {
sf_status recurrent_fwd(bool per_channel, sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* h0, const int32_t* cu_seqlens, int N, int B, int T, int H,
                        int HK, int K, int V, float scale, void* out, float* ht, void* state_pool, sf_dtype pool_dt,
                        int num_slots, long long slot_stride, const int32_t* state_indices,
                        const uint8_t* has_initial_state, void* stream) {
    const bool packed = cu_seqlens != nullptr;
    sf_status st = check_tokens(dt, B, T, H, HK, K, V, N, packed);
    if (st != SF_OK) return st;
    if (K != 64 && K != 128 && K != 256)
        return fail(SF_ERR_UNSUPPORTED, "the recurrent kernel is built for K in {64, 128, 256} (K=%d)", K);
    if (V % 32 != 0) return fail(SF_ERR_UNSUPPORTED, "V must be a multiple of 32 (V=%d)", V);
    if (!fits((long)N * H * (V / 32))) return fail(SF_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
    const bool paged = state_indices != nullptr;
    if (paged) {
        if (h0 || ht) return fail(SF_ERR_INVALID, "with state_indices the pool holds the states: h0 and ht must be NULL");
        if (pool_dt != SF_F32 && pool_dt != SF_BF16) return fail(SF_ERR_INVALID, "pool dtype must be SF_F32 or SF_BF16");
        if (num_slots < 0) return fail(SF_ERR_INVALID, "num_slots must not be negative");
        const long long block = (long long)H * V * K;
        if (slot_stride < block || slot_stride % 4 != 0)
            return fail(SF_ERR_INVALID, "slot_stride %lld must be a multiple of 4 and at least H*V*K = %lld",
                        slot_stride, block);
        if (!state_pool) return fail(SF_ERR_INVALID, "state_pool must not be NULL with state_indices");
        if (reinterpret_cast<uintptr_t>(state_pool) % 16 != 0) return fail(SF_ERR_INVALID, "state_pool must be 16-byte aligned");
    } else if (state_pool || has_initial_state) {
        return fail(SF_ERR_INVALID, "state_pool and has_initial_state need state_indices");
    }
    if (N == 0) return SF_OK;
    if ((long)B * T > 0 && (!q || !k || !v || !g || !beta || !out))  // (no tokens: nothing of them is read)
        return fail(SF_ERR_INVALID, "q, k, v, g, beta and out must not be NULL");
    if ((h0 && reinterpret_cast<uintptr_t>(h0) % 16 != 0) || (ht && reinterpret_cast<uintptr_t>(ht) % 16 != 0))
        return fail(SF_ERR_INVALID, "h0 and ht must be 16-byte aligned");
    if (per_channel && (reinterpret_cast<uintptr_t>(g) % 16 != 0))
        return fail(SF_ERR_INVALID, "the per-channel gate must be 16-byte aligned");
    hipError_t e = sf::launch_gdn_recurrent(dt == SF_BF16, paged && pool_dt == SF_BF16, q, k, v, g, beta, h0, ht,
                                            paged ? state_pool : nullptr, slot_stride, num_slots, state_indices,
                                            has_initial_state, cu_seqlens, N, T, H, HK, K, V, scale, out,
                                            static_cast<hipStream_t>(stream), per_channel);
    return hip_status(e, per_channel ? "sf_kda_recurrent_fwd launch" : "sf_gdn_recurrent_fwd launch");
}
}  // namespace

sf_status sf_gdn_recurrent_fwd(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* h0, const int32_t* cu_seqlens, int N, int B, int T,
                               int H, int HK, int K, int V, float scale, void* out, float* ht, void* state_pool,
                               sf_dtype pool_dt, int num_slots, long long slot_stride, const int32_t* state_indices,
                               const uint8_t* has_initial_state, void* stream) {
    return recurrent_fwd(false, dt, q, k, v, g, beta, h0, cu_seqlens, N, B, T, H, HK, K, V, scale, out, ht, state_pool,
                         pool_dt, num_slots, slot_stride, state_indices, has_initial_state, stream);
}

sf_status sf_kda_recurrent_fwd(sf_dtype dt, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* h0, const int32_t* cu_seqlens, int N, int B, int T,
                               int H, int K, int V, float scale, void* out, float* ht, void* state_pool,
                               sf_dtype pool_dt, int num_slots, long long slot_stride, const int32_t* state_indices,
                               const uint8_t* has_initial_state, void* stream) {
    if (!fits((long)B * T * H * K)) return fail(SF_ERR_UNSUPPORTED, "the gate has 2^31 or more elements");
    return recurrent_fwd(true, dt, q, k, v, g, beta, h0, cu_seqlens, N, B, T, H, H, K, V, scale, out, ht, state_pool,
                         pool_dt, num_slots, slot_stride, state_indices, has_initial_state, stream);
}

namespace {
sf_status decode_step(bool per_channel, int bounded, float lower_bound, sf_dtype dt, const void* packed_qkv,
                      const void* raw_gate, const void* raw_beta, const float* A_log, const float* dt_bias,
                      void* state_pool, sf_dtype pool_dt, int num_slots, long long slot_stride,
                      const int32_t* state_indices, const uint8_t* has_initial_state, int B, int H, int HK, int K,
                      int V, float scale, void* out, void* stream) {
    if (dt != SF_F32 && dt != SF_BF16) return fail(SF_ERR_INVALID, "dtype must be SF_F32 or SF_BF16");
    if (pool_dt != SF_F32 && pool_dt != SF_BF16) return fail(SF_ERR_INVALID, "pool dtype must be SF_F32 or SF_BF16");
    if (B < 0 || H <= 0 || HK <= 0 || K <= 0 || V <= 0 || num_slots < 0)
        return fail(SF_ERR_INVALID, "sizes must be positive (B=%d H=%d HK=%d K=%d V=%d num_slots=%d)", B, H, HK, K, V,
                    num_slots);
    if (H % HK != 0) return fail(SF_ERR_INVALID, "HK=%d must divide H=%d", HK, H);
    if (K != 64 && K != 128 && K != 256)
        return fail(SF_ERR_UNSUPPORTED, "decode is built for K in {64, 128, 256} (K=%d)", K);
    if (V % 16 != 0) return fail(SF_ERR_UNSUPPORTED, "V must be a multiple of 16 (V=%d)", V);
    const long long block = (long long)H * V * K;
    if (slot_stride < block || slot_stride % 4 != 0)
        return fail(SF_ERR_INVALID, "slot_stride %lld must be a multiple of 4 and at least H*V*K = %lld", slot_stride,
                    block);
    if (!fits((long)B * (2L * HK * K + (long)H * V)) || !fits((long)B * H * V) || B > kMaxElems / H)
        return fail(SF_ERR_UNSUPPORTED, "a tensor has 2^31 or more elements (int64 offsets are not supported)");
    if (B == 0) return SF_OK;
    if (!packed_qkv || !raw_gate || !raw_beta || !A_log || !dt_bias || !state_pool || !state_indices || !out)
        return fail(SF_ERR_INVALID, "packed_qkv, raw_gate, raw_beta, A_log, dt_bias, state_pool, state_indices and out "
                                    "must not be NULL");
    if (reinterpret_cast<uintptr_t>(state_pool) % 16 != 0 || reinterpret_cast<uintptr_t>(packed_qkv) % 16 != 0)
        return fail(SF_ERR_INVALID, "state_pool and packed_qkv must be 16-byte aligned");
    if (per_channel && (reinterpret_cast<uintptr_t>(dt_bias) % 16 != 0 ||
                        reinterpret_cast<uintptr_t>(raw_gate) % (dt == SF_BF16 ? 8 : 16) != 0))
        return fail(SF_ERR_INVALID, "dt_bias must be 16-byte and raw_gate %d-byte aligned", dt == SF_BF16 ? 8 : 16);
    hipError_t e = sf::launch_gdn_decode(dt == SF_BF16, pool_dt == SF_BF16, packed_qkv, raw_gate, raw_beta, A_log,
                                         dt_bias, state_pool, slot_stride, num_slots, state_indices,
                                         has_initial_state, B, H, HK, K, V, scale, out,
                                         static_cast<hipStream_t>(stream), per_channel, bounded, lower_bound);
    return hip_status(e, per_channel ? "sf_kda_decode launch" : "sf_gdn_decode launch");
}
}  // namespace

sf_status sf_gdn_decode(sf_dtype dt, const void* packed_qkv, const void* raw_gate, const void* raw_beta,
                        const float* A_log, const float* dt_bias, void* state_pool, sf_dtype pool_dt,
                        int num_slots, long long slot_stride, const int32_t* state_indices,
                        const uint8_t* has_initial_state, int B, int H, int HK, int K, int V, float scale,
                        void* out, void* stream) {
    return decode_step(false, 0, 0.f, dt, packed_qkv, raw_gate, raw_beta, A_log, dt_bias, state_pool, pool_dt,
                       num_slots, slot_stride, state_indices, has_initial_state, B, H, HK, K, V, scale, out, stream);
}

sf_status sf_kda_decode(sf_dtype dt, const void* packed_qkv, const void* raw_gate, const void* raw_beta,
                        const float* A_log, const float* dt_bias, sf_gate_kind kind, float lower_bound,
                        void* state_pool, sf_dtype pool_dt, int num_slots, long long slot_stride,
                        const int32_t* state_indices, const uint8_t* has_initial_state, int B, int H, int K, int V,
                        float scale, void* out, void* stream) {
    if (kind != SF_GATE_SOFTPLUS && kind != SF_GATE_BOUNDED)
        return fail(SF_ERR_INVALID, "kind must be SF_GATE_SOFTPLUS or SF_GATE_BOUNDED");
    if (kind == SF_GATE_BOUNDED && !(lower_bound <= 0.f && lower_bound > -3.0e38f))
        return fail(SF_ERR_INVALID, "the bounded kind needs a finite lower_bound <= 0 (got %g)", (double)lower_bound);
    return decode_step(true, kind == SF_GATE_BOUNDED ? 1 : 0, lower_bound, dt, packed_qkv, raw_gate, raw_beta, A_log,
                       dt_bias, state_pool, pool_dt, num_slots, slot_stride, state_indices, has_initial_state, B, H,
                       H, K, V, scale, out, stream);
}

}  // extern "C"

// Kimi Delta Attention chunk forward for gfx950 (attention-gym "Linear Attention", section "Kimi Delta
// Attention", chunk_kda): the delta rule with a per-channel gate, run per 64-token chunk with the StateFlow
// Section 2.2, Eq. (2) split.
//
// For one chunk of one (sequence, head) with entry state S [V x K] and, per key channel c, the within-chunk
// cumulative gate G_t[c] = sum_{i<=t} g_i[c] (Gamma_t = exp(G_t), a vector over the channels), the token rule
// (the state decays channel by channel, then the delta rule's correction and update, then the read) unrolls to
//   A_ts = beta_t sum_c k_t[c] k_s[c] exp(G_t[c] - G_s[c])   (s < t),   T = (I + A)^-1,
//   W = T diag(beta) (Gamma o K),   U = T diag(beta) V,   R = U - W S^T,
//   P_ts = scale sum_c q_t[c] k_s[c] exp(G_t[c] - G_s[c])   (s <= t),   Qg = scale (Gamma o Q),
//   O = Qg S^T + P R,
//   S' = S diag(Gamma_L) + R^T Kh,   Kh_s = exp(G_L - G_s) o k_s,
// where o multiplies each token row by its channel vector. Every exponent above is <= 0 (the cumulative
// gate only falls within a chunk), so the chunk form is exact for any finite, nonpositive gate: the decay
// between two tokens is applied per pair and channel rather than factored through exp(+G), which can
// overflow float32 for strong gates.
//
// Kernels (float32 arithmetic; q, k, v and the output in the input type):
//   kda_prep_kernel   per (chunk, head): W, U, P, Qg, Kh and Gamma_L into a record
//   kda_chain_kernel  per (sequence, head, 16-row slice of the state): the state chain and the output
#include "sf_device.h"
#include "sf_internal.h"

namespace sf {
namespace {

constexpr int BC = kGdnChunk;
constexpr int NT = 256;

// Record of one (chunk, head), floats: W [64][KD] | U [64][VD] | P [64][64] | Qg [64][KD] | Kh [64][KD] | Gamma_L [KD]
template <int KD>
struct KdaRec {
    static __host__ __device__ size_t w_off() { return 0; }
    static __host__ __device__ size_t u_off() { return (size_t)BC * KD; }
    static __host__ __device__ size_t p_off(int V) { return u_off() + (size_t)BC * V; }
    static __host__ __device__ size_t q_off(int V) { return p_off(V) + (size_t)BC * BC; }
    static __host__ __device__ size_t kh_off(int V) { return q_off(V) + (size_t)BC * KD; }
    static __host__ __device__ size_t gl_off(int V) { return kh_off(V) + (size_t)BC * KD; }
    static __host__ __device__ size_t floats(int V) { return gl_off(V) + KD; }
};

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
// float [ROWS][COLS + 1] through registers in 16-byte pieces, all of a thread's pieces in flight at once.
template <typename ST, int ROWS, int COLS>
struct Tile {
    static constexpr int E = 16 / (int)sizeof(ST);
    static constexpr int PPR = COLS / E;
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
// Prep: per (chunk slot, head). The per-channel cumulative gate (one thread per channel), A and P with the
// pairwise per-channel decays, T by forward substitution (one column per thread), then W, U, Qg, Kh.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD, int VD>
__global__ __launch_bounds__(NT) void kda_prep_kernel(const ST* __restrict__ q, const ST* __restrict__ k,
                                                      const ST* __restrict__ v, const float* __restrict__ g,
                                                      const float* __restrict__ beta, const int2* __restrict__ table,
                                                      const int32_t* __restrict__ cu, int T, int H, int nc, float scale,
                                                      float* __restrict__ rec) {
    typedef KdaRec<KD> RL;
    constexpr int LK = KD + 1, LL = BC + 1, LV = VD + 1;
    __shared__ float sK[BC * LK], sQ[BC * LK], sG[BC * LK];
    __shared__ float sA[BC * LL], sT[BC * LL];
    __shared__ float sB[BC];
    float* const sV = sQ;  // V rows replace Q rows once Qg and P are formed (VD <= KD)
    static_assert(VD <= KD, "V rows reuse the Q buffer");
    const int slot = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    int b, t0, L;
    if (!chunk_coords(slot, table, cu, T, nc, b, t0, L)) return;
    const long row0 = (long)b * T + t0;
    {
        Tile<ST, BC, KD> tk, tq;
        Tile<float, BC, KD> tg;
        tk.load(k + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tq.load(q + (row0 * H + h) * (long)KD, (long)H * KD, L);
        tg.load(g + (row0 * H + h) * (long)KD, (long)H * KD, L);  // padded tokens: g = 0
        tk.store(sK);
        tq.store(sQ);
        tg.store(sG);
    }
    if (tid < BC) sB[tid] = tid < L ? beta[(row0 + tid) * H + h] : 0.f;
    __syncthreads();
    // cumulative gate per channel, in place
    if (tid < KD) {
        float acc = 0.f;
        for (int t = 0; t < BC; ++t) {
            acc += sG[t * LK + tid];
            sG[t * LK + tid] = acc;
        }
    }
    __syncthreads();
    float* R = rec + ((size_t)slot * H + h) * RL::floats(VD);
    // A (strictly lower) into sA and P (lower with the diagonal) into the record; thread's entries (t, s) with
    // t = tid / 4, s = tid % 4 + 4 j
    const int t = tid >> 2, q4 = tid & 3;
    for (int j = 0; j < 16; ++j) {
        const int s2 = q4 + 4 * j;
        float a = 0.f, p = 0.f;
        if (s2 <= t)
            for (int c = 0; c < KD; ++c) {
                const float d = __expf(sG[t * LK + c] - sG[s2 * LK + c]) * sK[s2 * LK + c];
                a += sK[t * LK + c] * d;
                p += sQ[t * LK + c] * d;
            }
        sA[t * LL + s2] = s2 < t ? sB[t] * a : 0.f;
        R[RL::p_off(VD) + t * BC + s2] = s2 <= t ? scale * p : 0.f;
    }
    __syncthreads();
    // Qg = scale Gamma o Q and Kh = exp(G_L - G) o K to the record, then V rows into the Q buffer
    for (int i = tid; i < BC * KD; i += NT) {
        const int tt = i / KD, c = i % KD;
        const float G = sG[tt * LK + c], GL = sG[(BC - 1) * LK + c];
        R[RL::q_off(VD) + i] = scale * __expf(G) * sQ[tt * LK + c];
        R[RL::kh_off(VD) + i] = __expf(GL - G) * sK[tt * LK + c];
    }
    if (tid < KD) R[RL::gl_off(VD) + tid] = __expf(sG[(BC - 1) * LK + tid]);
    if (tid < BC) {
        // column j = tid of T = (I + A)^-1 (unit lower triangular): x_j = 1, x_t = -sum_{j<=s<t} A_ts x_s
        const int j = tid;
        for (int tt = 0; tt < BC; ++tt) {
            float x = tt == j ? 1.f : 0.f;
            if (tt > j)
                for (int s2 = j; s2 < tt; ++s2) x -= sA[tt * LL + s2] * sT[s2 * LL + j];
            sT[tt * LL + j] = x;
        }
    }
    __syncthreads();
    {
        Tile<ST, BC, VD> tv;
        tv.load(v + (row0 * H + h) * (long)VD, (long)H * VD, L);
        // (the Q rows are no longer read: Qg and P are in the record)
        float* dst = sV;
#pragma unroll
        for (int p = 0; p < Tile<ST, BC, VD>::PER; ++p) {
            const int idx = threadIdx.x + NT * p, row = idx / Tile<ST, BC, VD>::PPR,
                      col = (idx % Tile<ST, BC, VD>::PPR) * Tile<ST, BC, VD>::E;
            if (idx < Tile<ST, BC, VD>::PIECES)
#pragma unroll
                for (int e = 0; e < Tile<ST, BC, VD>::E; ++e)
                    dst[row * LV + col + e] = Elem<ST>::to_f(unit_of<ST>(tv.r[p], e));
        }
    }
    __syncthreads();
    // W[t][c] = sum_{s<=t} T[t][s] beta_s Gamma_s[c] K[s][c];  U[t][v] = sum_{s<=t} T[t][s] beta_s V[s][v]
    for (int m = 0; m < KD / 4; ++m) {
        const int c = q4 + 4 * m;
        float w = 0.f;
        for (int s2 = 0; s2 <= t; ++s2) w += sT[t * LL + s2] * sB[s2] * __expf(sG[s2 * LK + c]) * sK[s2 * LK + c];
        R[RL::w_off() + t * KD + c] = w;
    }
    for (int m = 0; m < VD / 4; ++m) {
        const int c = q4 + 4 * m;
        float u = 0.f;
        for (int s2 = 0; s2 <= t; ++s2) u += sT[t * LL + s2] * sB[s2] * sV[s2 * LV + c];
        R[RL::u_off() + t * VD + c] = u;
    }
}

// ---------------------------------------------------------------------------------------------------------
// Chain: one 16-row slice of the state of one (sequence, head) through its chunks; the next chunk's record
// tiles load while the current one computes. Thread owns state entries e = tid + 256 m.
// ---------------------------------------------------------------------------------------------------------
template <typename ST, int KD, int VD>
__global__ __launch_bounds__(NT) void kda_chain_kernel(const float* __restrict__ h0, const int32_t* __restrict__ cu,
                                                       const int* __restrict__ chunk_off, const float* __restrict__ rec,
                                                       int T, int H, int n_seq, int nc, int nvs, ST* __restrict__ out,
                                                       float* __restrict__ ht) {
    typedef KdaRec<KD> RL;
    constexpr int LK = KD + 1, LL = BC + 1, LV = 17, NE = 16 * KD / NT;
    __shared__ float sW[BC * LK], sQg[BC * LK], sKh[BC * LK], sP[BC * LL], sU[BC * LV], sR[BC * LV], sS[16 * LK];
    __shared__ float sGL[KD];
    int chain, vs;
    xcd_split(blockIdx.x, nvs, chain, vs);
    if (chain >= n_seq * H) return;
    const int n = chain / H, h = chain % H, tid = threadIdx.x, v0 = 16 * vs;
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
    const int nch = (eos - bos + BC - 1) / BC;
    float S[NE];
#pragma unroll
    for (int m = 0; m < NE; ++m) {
        const int e = tid + NT * m;
        S[m] = h0 ? h0[(((size_t)n * H + h) * VD + v0 + e / KD) * KD + e % KD] : 0.f;
    }
    Tile<float, BC, KD> tw, tq, tk;
    Tile<float, BC, BC> tp;
    Tile<float, BC, 16> tu;
    float gl = 0.f;
    auto issue = [&](int ci) __attribute__((always_inline)) {
        const float* R = rec + ((size_t)(slot0 + ci) * H + h) * RL::floats(VD);
        tw.load(R + RL::w_off(), KD, BC);
        tq.load(R + RL::q_off(VD), KD, BC);
        tk.load(R + RL::kh_off(VD), KD, BC);
        tp.load(R + RL::p_off(VD), BC, BC);
        tu.load(R + RL::u_off() + v0, VD, BC);
        gl = tid < KD ? R[RL::gl_off(VD) + tid] : 0.f;
    };
    if (nch > 0) issue(0);
    const int t = tid >> 2, v4 = (tid & 3) * 4;
    for (int ci = 0; ci < nch; ++ci) {
        const long row0 = (long)b * T + bos + (long)ci * BC;
        const int L = min(BC, eos - (bos + ci * BC));
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + NT * m;
            sS[(e / KD) * LK + e % KD] = S[m];
        }
        tw.store(sW);
        tq.store(sQg);
        tk.store(sKh);
        tp.store(sP);
        tu.store(sU);
        if (tid < KD) sGL[tid] = gl;
        __syncthreads();
        if (ci + 1 < nch) issue(ci + 1);
        // R = U - W S^T and QS = Qg S^T on (token t, values v4 .. v4 + 3)
        float r[4], qs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[j] = sU[t * LV + v4 + j];
            qs[j] = 0.f;
        }
        for (int c = 0; c < KD; ++c) {
            const float w = sW[t * LK + c], qg = sQg[t * LK + c];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sv = sS[(v4 + j) * LK + c];
                r[j] -= w * sv;
                qs[j] += qg * sv;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sR[t * LV + v4 + j] = r[j];
        __syncthreads();
        // O = Qg S^T + P R
        float o[4] = {qs[0], qs[1], qs[2], qs[3]};
        for (int s2 = 0; s2 <= t; ++s2) {
            const float p = sP[t * LL + s2];
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] += p * sR[s2 * LV + v4 + j];
        }
        if (t < L)
#pragma unroll
            for (int j = 0; j < 4; ++j) out[((row0 + t) * H + h) * (long)VD + v0 + v4 + j] = Elem<ST>::from_f(o[j]);
        // S <- S diag(Gamma_L) + R^T Kh
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + NT * m, rr = e / KD, c = e % KD;
            float acc = S[m] * sGL[c];
            for (int tt = 0; tt < BC; ++tt) acc += sR[tt * LV + rr] * sKh[tt * LK + c];
            S[m] = acc;
        }
        __syncthreads();
    }
    if (ht) {
#pragma unroll
        for (int m = 0; m < NE; ++m) {
            const int e = tid + NT * m;
            ht[(((size_t)n * H + h) * VD + v0 + e / KD) * KD + e % KD] = S[m];
        }
    }
}

template <typename ST, int KD, int VD>
hipError_t run_kda(const ST* q, const ST* k, const ST* v, const float* g, const float* beta, const float* h0,
                   const int32_t* cu, const KdaWorkspace& ws, int N, int B, int T, int H, float scale, ST* out,
                   float* ht, hipStream_t s) {
    const bool packed = cu != nullptr;
    const long slots = gdn_slots(B, T, N, packed);
    const int nc = (T + BC - 1) / BC;
    hipError_t err;
    if (packed) {
        err = launch_chunk_table(cu, N, BC, slots, ws.chunk_off, ws.table, s);
        if (err != hipSuccess) return err;
    }
    if (slots > 0) {
        timing_begin("kda_prep", s);
        kda_prep_kernel<ST, KD, VD><<<dim3((unsigned)slots, H), NT, 0, s>>>(q, k, v, g, beta, packed ? ws.table : nullptr,
                                                                           cu, T, H, nc, scale, ws.rec);
        timing_end(s);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const long chains = (long)N * H;
    if (chains == 0) return hipSuccess;
    const int nvs = VD / 16;
    const unsigned grid = (unsigned)(((chains + 7) / 8) * 8 * nvs);
    timing_begin("kda_chain", s);
    kda_chain_kernel<ST, KD, VD><<<grid, NT, 0, s>>>(h0, cu, ws.chunk_off, ws.rec, T, H, N, nc, nvs, out, ht);
    timing_end(s);
    return hipGetLastError();
}

}  // namespace

size_t kda_record_floats(int K, int V) {
    return K == 128 ? KdaRec<128>::floats(V) : KdaRec<64>::floats(V);
}

hipError_t launch_kda_chunk(bool bf16, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* h0, const int32_t* cu, const KdaWorkspace& ws, int N,
                            int B, int T, int H, int K, int V, float scale, void* out, float* ht, hipStream_t s) {
#define SF_KDA_RUN(E, KK, VV)                                                                                      \
    return run_kda<E, KK, VV>(static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), g, beta, \
                              h0, cu, ws, N, B, T, H, scale, static_cast<E*>(out), ht, s)
    if (bf16) {
        if (K == 128 && V == 128) SF_KDA_RUN(bf16_t, 128, 128);
        if (K == 128 && V == 64) SF_KDA_RUN(bf16_t, 128, 64);
        SF_KDA_RUN(bf16_t, 64, 64);
    }
    if (K == 128 && V == 128) SF_KDA_RUN(float, 128, 128);
    if (K == 128 && V == 64) SF_KDA_RUN(float, 128, 64);
    SF_KDA_RUN(float, 64, 64);
#undef SF_KDA_RUN
}

}  // namespace sf

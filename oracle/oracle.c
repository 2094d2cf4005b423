/*
 * Oracle for the chunked linear recurrence forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path loads this file:
 * only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * build, load or call it. It shares no code, header, table or helper with
 * the HIP library, and it never reads anything the HIP path produced.
 *
 * Everything here is plain, slow and written to be checked by eye against
 * the pages it follows:
 *   [GDN]   attention-gym "Linear Attention" page, section "Gated Delta Rule":
 *           the per-token rule (decay the state by exp(gate), form the
 *           beta-scaled residual against the decayed state, add its outer
 *           product with the key, read the updated state with the scaled
 *           query) and the [N, H, V, K] state layout, grouped q/k heads,
 *           cu_seqlens packing with empty sequences passing their state.
 *   [EQ1]   "StateFlow: Sequence Pipeline Parallelism for Long-Context
 *           Modeling with Linear Recurrence", Section 2.1, Eq. (1): the
 *           general linear recurrence S_t = S_{t-1} F_t + v_t k_t^T,
 *           y_t = S_t q_t; for Mamba-2 F_t is a scalar times the identity.
 *   [CP]    attention-gym "Linear Attention" page, section "Context
 *           Parallelism": every range of tokens is an affine map of its
 *           entry state, S_out = S_in @ A + B; sub-section "cuDNN local
 *           execution": B is the final state from a zero entry, A the final
 *           state from an identity entry with the value term disabled, and
 *           an empty range gives the identity map.
 *   [SSD]   Megatron-LM pull request "Mamba2 state-passing context
 *           parallelism": S_out = a_block * S_in + S_ext per causal segment,
 *           true entry states recovered by an exclusive causal scan.
 *   [EQ2]   StateFlow Section 2.2, Eq. (2): the Pre / ST / Out chunk split
 *           (only used by the chunked self-check functions below).
 *
 * Precision: inputs arrive as float32 arrays (bf16 inputs are widened
 * exactly by the caller); all arithmetic and every output is float64, except
 * orc_forward_f32, a float32 build of the two token loops that serves only as
 * the CPU throughput baseline (never as a parity reference).
 *
 * Parity pins: every exported function is pinned by tests/test_oracle.py
 * against closed forms, brute force or invariants that do not reuse this
 * code (see the header of that file for the list).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Token range [*bos, *eos) and batch row of logical sequence n. Without
 * cu_seqlens every batch row is one sequence of length T; with cu_seqlens the
 * input is batch-one and sequence n covers [cu[n], cu[n+1]) ([GDN], cu_seqlens
 * parameter). */
static void seq_range(const int32_t *cu, int n, int T, int *b, int *bos, int *eos)
{
    if (cu) {
        *b = 0;
        *bos = cu[n];
        *eos = cu[n + 1];
    } else {
        *b = n;
        *bos = 0;
        *eos = T;
    }
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* ---------------------------------------------------------------------------
 * One Gated Delta Rule chain ([GDN]), token by token, on a state of `rows`
 * rows and K columns. Row r of the state uses value column r of v when
 * use_values is set, and value 0 otherwise (the "value term disabled" probe
 * of [CP]). If o is not NULL, o[t][r] = scale * (S_t q_t)[r] for the first
 * `orows` rows.
 *   S      [rows][K]   in: entry state, out: exit state
 *   qs,ks  token stride of q/k (elements), vs token stride of v,
 *   gs     token stride of g and beta, os token stride of o.
 * ------------------------------------------------------------------------- */
static void gdn_chain(double *S, int rows, int K,
                      const float *q, const float *k, const float *v,
                      const float *g, const float *beta,
                      long qs, long vs, long gs, int ntok, int use_values,
                      double scale, double *o, long os, int orows)
{
    double *r = (double *)malloc(sizeof(double) * (size_t)rows);
    for (int t = 0; t < ntok; ++t) {
        const float *kt = k + (long)t * qs;
        const double gam = exp((double)g[(long)t * gs]);
        const double bt = (double)beta[(long)t * gs];
        /* decayed_state = exp(gate) * state */
        for (long i = 0; i < (long)rows * K; ++i)
            S[i] *= gam;
        /* residual = beta * (value - decayed_state @ key) */
        for (int row = 0; row < rows; ++row) {
            double dk = 0.0;
            for (int c = 0; c < K; ++c)
                dk += S[(long)row * K + c] * (double)kt[c];
            double val = use_values ? (double)v[(long)t * vs + row] : 0.0;
            r[row] = bt * (val - dk);
        }
        /* state = decayed_state + outer(residual, key) */
        for (int row = 0; row < rows; ++row)
            for (int c = 0; c < K; ++c)
                S[(long)row * K + c] += r[row] * (double)kt[c];
        /* output = scale * state @ query */
        if (o) {
            const float *qt = q + (long)t * qs;
            for (int row = 0; row < orows; ++row) {
                double acc = 0.0;
                for (int c = 0; c < K; ++c)
                    acc += S[(long)row * K + c] * (double)qt[c];
                o[(long)t * os + row] = scale * acc;
            }
        }
    }
    free(r);
}

/* Gated Delta Rule forward ([GDN]).
 *   q, k  [B, T, HK, K] float32;  v [B, T, H, V];  g, beta [B, T, H]
 *   h0    [N, H, V, K] float32 or NULL (zero entry state)
 *   cu    int32 [N + 1] or NULL (then N == B)
 *   out   [B, T, H, V] float64: rows outside every sequence are left as given
 *   ht    [N, H, V, K] float64 or NULL
 * Value head h reads q/k head h / (H / HK). */
void orc_gdn_forward(const float *q, const float *k, const float *v,
                     const float *g, const float *beta, const float *h0,
                     const int32_t *cu, int N, int B, int T, int H, int HK,
                     int K, int V, double scale, double *out, double *ht,
                     int nthreads)
{
    (void)B;
    set_threads(nthreads);
    const int grp = H / HK;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int h = 0; h < H; ++h) {
            int b, bos, eos;
            seq_range(cu, n, T, &b, &bos, &eos);
            const int hk = h / grp;
            double *S = (double *)calloc((size_t)V * K, sizeof(double));
            if (h0)
                for (long i = 0; i < (long)V * K; ++i)
                    S[i] = (double)h0[((long)n * H + h) * V * K + i];
            const long tok0 = (long)b * T + bos;
            gdn_chain(S, V, K,
                      q + (tok0 * HK + hk) * K, k + (tok0 * HK + hk) * K,
                      v + (tok0 * H + h) * V, g + tok0 * H + h, beta + tok0 * H + h,
                      (long)HK * K, (long)H * V, H, eos - bos, 1, scale,
                      out + (tok0 * H + h) * V, (long)H * V, V);
            if (ht)
                memcpy(ht + ((long)n * H + h) * V * K, S, sizeof(double) * V * K);
            free(S);
        }
    }
}

/* Gated Delta Rule segment summary by probing ([CP], "cuDNN local
 * execution"): for every range (sequence of the same indexing as
 * orc_gdn_forward) S_ext = final state from a zero entry state, and
 * M = final state from the K x K identity entry with the value term
 * disabled. Then for every entry state S_in, exit = S_in @ M + S_ext.
 *   M [N, H, K, K], S_ext [N, H, V, K] float64. */
void orc_gdn_summary(const float *k, const float *v, const float *g,
                     const float *beta, const int32_t *cu, int N, int B, int T,
                     int H, int HK, int K, int V, double *M, double *S_ext,
                     int nthreads)
{
    (void)B;
    set_threads(nthreads);
    const int grp = H / HK;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int h = 0; h < H; ++h) {
            int b, bos, eos;
            seq_range(cu, n, T, &b, &bos, &eos);
            const int hk = h / grp;
            const long tok0 = (long)b * T + bos;
            const float *kp = k + (tok0 * HK + hk) * K;
            const float *vp = v + (tok0 * H + h) * V;
            const float *gp = g + tok0 * H + h;
            const float *bp = beta + tok0 * H + h;
            /* B: zero entry, values on */
            double *Sb = S_ext + ((long)n * H + h) * V * K;
            memset(Sb, 0, sizeof(double) * V * K);
            gdn_chain(Sb, V, K, NULL, kp, vp, gp, bp, (long)HK * K, (long)H * V, H,
                      eos - bos, 1, 0.0, NULL, 0, 0);
            /* A: identity entry, value term disabled */
            double *Sa = M + ((long)n * H + h) * K * K;
            memset(Sa, 0, sizeof(double) * K * K);
            for (int i = 0; i < K; ++i)
                Sa[(long)i * K + i] = 1.0;
            gdn_chain(Sa, K, K, NULL, kp, vp, gp, bp, (long)HK * K, (long)H * V, H,
                      eos - bos, 0, 0.0, NULL, 0, 0);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Scalar-gated linear attention ([EQ1] with F_t = exp(g_t) I, as in the SSD
 * page [SSD]): S_t = exp(g_t) S_{t-1} + v_t k_t^T, o_t = scale * S_t q_t.
 * Same layouts and indexing as orc_gdn_forward (no beta).
 * ------------------------------------------------------------------------- */
static void gla_chain(double *S, int V, int K, const float *q, const float *k,
                      const float *v, const float *g, long qs, long vs, long gs,
                      int ntok, double scale, double *o, long os)
{
    for (int t = 0; t < ntok; ++t) {
        const float *kt = k + (long)t * qs;
        const float *vt = v + (long)t * vs;
        const double gam = exp((double)g[(long)t * gs]);
        for (int row = 0; row < V; ++row)
            for (int c = 0; c < K; ++c)
                S[(long)row * K + c] = gam * S[(long)row * K + c] +
                                       (double)vt[row] * (double)kt[c];
        if (o) {
            const float *qt = q + (long)t * qs;
            for (int row = 0; row < V; ++row) {
                double acc = 0.0;
                for (int c = 0; c < K; ++c)
                    acc += S[(long)row * K + c] * (double)qt[c];
                o[(long)t * os + row] = scale * acc;
            }
        }
    }
}

void orc_gla_forward(const float *q, const float *k, const float *v,
                     const float *g, const float *h0, const int32_t *cu, int N,
                     int B, int T, int H, int HK, int K, int V, double scale,
                     double *out, double *ht, int nthreads)
{
    (void)B;
    set_threads(nthreads);
    const int grp = H / HK;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int h = 0; h < H; ++h) {
            int b, bos, eos;
            seq_range(cu, n, T, &b, &bos, &eos);
            const int hk = h / grp;
            double *S = (double *)calloc((size_t)V * K, sizeof(double));
            if (h0)
                for (long i = 0; i < (long)V * K; ++i)
                    S[i] = (double)h0[((long)n * H + h) * V * K + i];
            const long tok0 = (long)b * T + bos;
            gla_chain(S, V, K, q + (tok0 * HK + hk) * K, k + (tok0 * HK + hk) * K,
                      v + (tok0 * H + h) * V, g + tok0 * H + h, (long)HK * K,
                      (long)H * V, H, eos - bos, scale, out + (tok0 * H + h) * V,
                      (long)H * V);
            if (ht)
                memcpy(ht + ((long)n * H + h) * V * K, S, sizeof(double) * V * K);
            free(S);
        }
    }
}

/* Scalar-gate summary ([SSD]): S_ext = final state from a zero entry,
 * a_block = exp(sum of the range's gates), so S_out = a_block * S_in + S_ext.
 *   a [N, H], S_ext [N, H, V, K] float64. */
void orc_gla_summary(const float *k, const float *v, const float *g,
                     const int32_t *cu, int N, int B, int T, int H, int HK,
                     int K, int V, double *a, double *S_ext, int nthreads)
{
    (void)B;
    set_threads(nthreads);
    const int grp = H / HK;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int h = 0; h < H; ++h) {
            int b, bos, eos;
            seq_range(cu, n, T, &b, &bos, &eos);
            const int hk = h / grp;
            const long tok0 = (long)b * T + bos;
            double *Sb = S_ext + ((long)n * H + h) * V * K;
            memset(Sb, 0, sizeof(double) * V * K);
            gla_chain(Sb, V, K, NULL, k + (tok0 * HK + hk) * K, v + (tok0 * H + h) * V,
                      g + tok0 * H + h, (long)HK * K, (long)H * V, H, eos - bos, 0.0,
                      NULL, 0);
            double sg = 0.0;
            for (int t = bos; t < eos; ++t)
                sg += (double)g[((long)b * T + t) * H + h];
            a[(long)n * H + h] = exp(sg);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Exclusive state scan over segment summaries ([SSD] "exclusive causal
 * scan"; [CP] composition of affine maps). Segment row s = b * n_seg + j.
 *   kind 0 (delta rule): S_in[b,0] = h0[b] (or 0),
 *                        S_in[b,j+1] = S_in[b,j] @ M[b,j] + S_ext[b,j]
 *   kind 1 (scalar gate): S_in[b,j+1] = a[b,j] * S_in[b,j] + S_ext[b,j]
 *   M: kind 0 [B*n_seg, H, K, K]; kind 1 a [B*n_seg, H]
 *   S_ext, S_in [B*n_seg, H, V, K]; h0, S_final [B, H, V, K] (h0 may be NULL,
 *   S_final may be NULL). All float64.
 * ------------------------------------------------------------------------- */
void orc_state_scan(int kind, const double *M, const double *S_ext,
                    const double *h0, int B, int n_seg, int H, int K, int V,
                    double *S_in, double *S_final)
{
    const long VK = (long)V * K;
    double *cur = (double *)malloc(sizeof(double) * VK);
    double *nxt = (double *)malloc(sizeof(double) * VK);
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            for (long i = 0; i < VK; ++i)
                cur[i] = h0 ? h0[((long)b * H + h) * VK + i] : 0.0;
            for (int j = 0; j < n_seg; ++j) {
                const long s = (long)b * n_seg + j;
                memcpy(S_in + (s * H + h) * VK, cur, sizeof(double) * VK);
                const double *E = S_ext + (s * H + h) * VK;
                if (kind == 0) {
                    const double *Mj = M + (s * H + h) * (long)K * K;
                    for (int r = 0; r < V; ++r)
                        for (int c = 0; c < K; ++c) {
                            double acc = 0.0;
                            for (int i = 0; i < K; ++i)
                                acc += cur[(long)r * K + i] * Mj[(long)i * K + c];
                            nxt[(long)r * K + c] = acc + E[(long)r * K + c];
                        }
                } else {
                    const double a = M[s * H + h];
                    for (long i = 0; i < VK; ++i)
                        nxt[i] = a * cur[i] + E[i];
                }
                double *tmp = cur;
                cur = nxt;
                nxt = tmp;
            }
            if (S_final)
                memcpy(S_final + ((long)b * H + h) * VK, cur, sizeof(double) * VK);
        }
    }
    free(cur);
    free(nxt);
}

/* ---------------------------------------------------------------------------
 * Chunked forms, used ONLY to check that the chunk algebra reproduces the
 * token recurrence ("chunking changes only the decomposition and
 * floating-point order", [GDN] chunk_gdn). Never a reference for the GPU.
 *
 * For one chunk of L tokens with entry state S [V x K] ([EQ2] Pre/ST/Out):
 *   G = within-chunk cumulative sum of the gates
 *   A[t][i] = beta_t exp(G_t - G_i) (k_t . k_i) for i < t,  T = (I + A)^-1
 *   W = T diag(beta exp(G)) K,  U = T diag(beta) V
 *   R = U - W S^T                        (corrected values, V^new of Eq. 2)
 *   O = scale (diag(exp G) Q S^T + (D o Q K^T) R),  D[t][i] = exp(G_t - G_i), i <= t
 *   S' = exp(G_L) S + sum_t exp(G_L - G_t) r_t k_t^T
 * Scalar gate: R = V, no solve.
 * ------------------------------------------------------------------------- */
static void chunked_chain(int delta, double *S, int V, int K, int C,
                          const float *q, const float *k, const float *v,
                          const float *g, const float *beta, long qs, long vs,
                          long gs, int ntok, double scale, double *o, long os)
{
    double *G = (double *)malloc(sizeof(double) * C);
    double *A = (double *)malloc(sizeof(double) * C * C);
    double *Tm = (double *)malloc(sizeof(double) * C * C);
    double *R = (double *)malloc(sizeof(double) * C * V);
    double *Snew = (double *)malloc(sizeof(double) * V * K);
    for (int c0 = 0; c0 < ntok; c0 += C) {
        const int L = (ntok - c0 < C) ? ntok - c0 : C;
        double acc = 0.0;
        for (int t = 0; t < L; ++t) {
            acc += (double)g[(long)(c0 + t) * gs];
            G[t] = acc;
        }
#define KK(t, c) ((double)k[(long)(c0 + (t)) * qs + (c)])
#define QQ(t, c) ((double)q[(long)(c0 + (t)) * qs + (c)])
#define VV(t, r) ((double)v[(long)(c0 + (t)) * vs + (r)])
#define BB(t) ((double)beta[(long)(c0 + (t)) * gs])
        if (delta) {
            for (int t = 0; t < L; ++t)
                for (int i = 0; i < L; ++i) {
                    double a = 0.0;
                    if (i < t) {
                        double kk = 0.0;
                        for (int c = 0; c < K; ++c)
                            kk += KK(t, c) * KK(i, c);
                        a = BB(t) * exp(G[t] - G[i]) * kk;
                    }
                    A[t * C + i] = a;
                }
            /* T = (I + A)^-1 by forward substitution, column by column */
            for (int j = 0; j < L; ++j)
                for (int t = 0; t < L; ++t) {
                    double s = (t == j) ? 1.0 : 0.0;
                    for (int i = 0; i < t; ++i)
                        s -= A[t * C + i] * Tm[i * C + j];
                    Tm[t * C + j] = s;
                }
            /* R = T diag(beta) V - T diag(beta exp(G)) K S^T */
            for (int t = 0; t < L; ++t)
                for (int r = 0; r < V; ++r) {
                    double u = 0.0;
                    for (int i = 0; i < L; ++i) {
                        double ks = 0.0;
                        for (int c = 0; c < K; ++c)
                            ks += KK(i, c) * S[(long)r * K + c];
                        u += Tm[t * C + i] * BB(i) * (VV(i, r) - exp(G[i]) * ks);
                    }
                    R[t * V + r] = u;
                }
        } else {
            for (int t = 0; t < L; ++t)
                for (int r = 0; r < V; ++r)
                    R[t * V + r] = VV(t, r);
        }
        if (o) {
            for (int t = 0; t < L; ++t)
                for (int r = 0; r < V; ++r) {
                    double qs_ = 0.0;
                    for (int c = 0; c < K; ++c)
                        qs_ += QQ(t, c) * S[(long)r * K + c];
                    double intra = 0.0;
                    for (int i = 0; i <= t; ++i) {
                        double qk = 0.0;
                        for (int c = 0; c < K; ++c)
                            qk += QQ(t, c) * KK(i, c);
                        intra += exp(G[t] - G[i]) * qk * R[i * V + r];
                    }
                    o[(long)(c0 + t) * os + r] = scale * (exp(G[t]) * qs_ + intra);
                }
        }
        for (int r = 0; r < V; ++r)
            for (int c = 0; c < K; ++c) {
                double s = exp(G[L - 1]) * S[(long)r * K + c];
                for (int t = 0; t < L; ++t)
                    s += exp(G[L - 1] - G[t]) * R[t * V + r] * KK(t, c);
                Snew[(long)r * K + c] = s;
            }
        memcpy(S, Snew, sizeof(double) * V * K);
#undef KK
#undef QQ
#undef VV
#undef BB
    }
    free(G);
    free(A);
    free(Tm);
    free(R);
    free(Snew);
}

/* delta = 1: Gated Delta Rule; delta = 0: scalar-gated linear attention
 * (beta ignored, may be NULL). Same layouts as orc_gdn_forward. */
void orc_chunked_forward(int delta, int C, const float *q, const float *k,
                         const float *v, const float *g, const float *beta,
                         const float *h0, const int32_t *cu, int N, int B, int T,
                         int H, int HK, int K, int V, double scale, double *out,
                         double *ht, int nthreads)
{
    (void)B;
    set_threads(nthreads);
    const int grp = H / HK;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int h = 0; h < H; ++h) {
            int b, bos, eos;
            seq_range(cu, n, T, &b, &bos, &eos);
            const int hk = h / grp;
            double *S = (double *)calloc((size_t)V * K, sizeof(double));
            if (h0)
                for (long i = 0; i < (long)V * K; ++i)
                    S[i] = (double)h0[((long)n * H + h) * V * K + i];
            const long tok0 = (long)b * T + bos;
            chunked_chain(delta, S, V, K, C, q + (tok0 * HK + hk) * K,
                          k + (tok0 * HK + hk) * K, v + (tok0 * H + h) * V,
                          g + tok0 * H + h, delta ? beta + tok0 * H + h : NULL,
                          (long)HK * K, (long)H * V, H, eos - bos, scale,
                          out + (tok0 * H + h) * V, (long)H * V);
            if (ht)
                memcpy(ht + ((long)n * H + h) * V * K, S, sizeof(double) * V * K);
            free(S);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Float32 builds of the two token loops above: the same steps in the same
 * order with float arithmetic (expf). They are the CPU throughput baseline
 * only; parity always uses the float64 functions.
 * ------------------------------------------------------------------------- */
static void gdn_chain_f32(float *S, int V, int K, const float *q, const float *k,
                          const float *v, const float *g, const float *beta,
                          long qs, long vs, long gs, int ntok, float scale,
                          float *o, long os)
{
    float *r = (float *)malloc(sizeof(float) * (size_t)V);
    for (int t = 0; t < ntok; ++t) {
        const float *kt = k + (long)t * qs;
        const float gam = expf(g[(long)t * gs]);
        const float bt = beta[(long)t * gs];
        for (long i = 0; i < (long)V * K; ++i)
            S[i] *= gam;
        for (int row = 0; row < V; ++row) {
            float dk = 0.f;
            for (int c = 0; c < K; ++c)
                dk += S[(long)row * K + c] * kt[c];
            r[row] = bt * (v[(long)t * vs + row] - dk);
        }
        for (int row = 0; row < V; ++row)
            for (int c = 0; c < K; ++c)
                S[(long)row * K + c] += r[row] * kt[c];
        const float *qt = q + (long)t * qs;
        for (int row = 0; row < V; ++row) {
            float acc = 0.f;
            for (int c = 0; c < K; ++c)
                acc += S[(long)row * K + c] * qt[c];
            o[(long)t * os + row] = scale * acc;
        }
    }
    free(r);
}

static void gla_chain_f32(float *S, int V, int K, const float *q, const float *k,
                          const float *v, const float *g, long qs, long vs, long gs,
                          int ntok, float scale, float *o, long os)
{
    for (int t = 0; t < ntok; ++t) {
        const float *kt = k + (long)t * qs;
        const float *vt = v + (long)t * vs;
        const float gam = expf(g[(long)t * gs]);
        for (int row = 0; row < V; ++row)
            for (int c = 0; c < K; ++c)
                S[(long)row * K + c] = gam * S[(long)row * K + c] + vt[row] * kt[c];
        const float *qt = q + (long)t * qs;
        for (int row = 0; row < V; ++row) {
            float acc = 0.f;
            for (int c = 0; c < K; ++c)
                acc += S[(long)row * K + c] * qt[c];
            o[(long)t * os + row] = scale * acc;
        }
    }
}

/* kind 1: Gated Delta Rule (beta used), kind 0: scalar gate. Layouts as
 * orc_gdn_forward, with float32 out [B, T, H, V] and ht [N, H, V, K]. */
void orc_forward_f32(int delta, const float *q, const float *k, const float *v,
                     const float *g, const float *beta, const float *h0,
                     const int32_t *cu, int N, int B, int T, int H, int HK, int K,
                     int V, float scale, float *out, float *ht, int nthreads)
{
    (void)B;
    set_threads(nthreads);
    const int grp = H / HK;
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int h = 0; h < H; ++h) {
            int b, bos, eos;
            seq_range(cu, n, T, &b, &bos, &eos);
            const int hk = h / grp;
            float *S = (float *)calloc((size_t)V * K, sizeof(float));
            if (h0)
                memcpy(S, h0 + ((long)n * H + h) * V * K, sizeof(float) * V * K);
            const long tok0 = (long)b * T + bos;
            if (delta)
                gdn_chain_f32(S, V, K, q + (tok0 * HK + hk) * K, k + (tok0 * HK + hk) * K,
                              v + (tok0 * H + h) * V, g + tok0 * H + h, beta + tok0 * H + h,
                              (long)HK * K, (long)H * V, H, eos - bos, scale,
                              out + (tok0 * H + h) * V, (long)H * V);
            else
                gla_chain_f32(S, V, K, q + (tok0 * HK + hk) * K, k + (tok0 * HK + hk) * K,
                              v + (tok0 * H + h) * V, g + tok0 * H + h, (long)HK * K,
                              (long)H * V, H, eos - bos, scale, out + (tok0 * H + h) * V,
                              (long)H * V);
            if (ht)
                memcpy(ht + ((long)n * H + h) * V * K, S, sizeof(float) * V * K);
            free(S);
        }
    }
}

/* ---------------------------------------------------------------------------
 * Gated Delta Rule backward ([GDN] token rule, differentiated by reverse-mode
 * through the token loop; the state cotangent is carried from the last token
 * back to the entry state, as StateFlow Section 2.2, Eq. (6)-(7) carries the
 * gradient of the recurrence backwards through the chunks).
 *
 * Loss convention: the caller's upstream gradients are do = dLoss/do_t
 * [B, T, H, V] and dht = dLoss/dht [N, H, V, K] (NULL: zero). The outputs are
 * the gradients of the same loss with respect to every input:
 *   dq, dk [B, T, HK, K] (summed over the H/HK value heads of a q/k head),
 *   dv [B, T, H, V], dg, dbeta [B, T, H], dh0 [N, H, V, K] (NULL: skipped),
 * all float64; entries of tokens outside every sequence are left as given.
 *
 * For one token, with gamma = exp(g) and the forward rule
 *   D = gamma S_prev;  u = v - D k;  r = beta u;  S = D + r k^T;  o = scale S q,
 * and dS the gradient with respect to S (all later use of S included):
 *   dS += scale do q^T;   dq = scale S^T do
 *   dr = dS k;            dk = dS^T r
 *   du = beta dr;         dbeta = dr . u;   dv = du
 *   dD = dS - du k^T;     dk -= D^T du
 *   dg = gamma <dD, S_prev>;  and the gradient of S_prev is gamma dD.
 * The states S_prev of the reverse sweep are recomputed with the forward rule
 * from a checkpoint every BWD_BLOCK tokens.
 * ------------------------------------------------------------------------- */
#define BWD_BLOCK 64

/* One token of the [GDN] rule on S [V][K] (in place). */
static void gdn_token(double *S, int V, int K, const float *kt, const float *vt,
                      double gam, double bt)
{
    for (long i = 0; i < (long)V * K; ++i)
        S[i] *= gam;
    for (int row = 0; row < V; ++row) {
        double dk = 0.0;
        for (int c = 0; c < K; ++c)
            dk += S[(long)row * K + c] * (double)kt[c];
        const double rr = bt * ((double)vt[row] - dk);
        for (int c = 0; c < K; ++c)
            S[(long)row * K + c] += rr * (double)kt[c];
    }
}

void orc_gdn_backward(const float *q, const float *k, const float *v,
                      const float *g, const float *beta, const float *h0,
                      const float *dout, const float *dht, const int32_t *cu,
                      int N, int B, int T, int H, int HK, int K, int V,
                      double scale, double *dq, double *dk, double *dv,
                      double *dg, double *dbeta, double *dh0, int nthreads)
{
    (void)B;
    set_threads(nthreads);
    const int grp = H / HK;
    /* one (sequence, q/k head) per task: its value heads accumulate into the
     * same dq, dk rows one after the other */
    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int n = 0; n < N; ++n) {
        for (int hk = 0; hk < HK; ++hk) {
            int b, bos, eos;
            seq_range(cu, n, T, &b, &bos, &eos);
            const int ntok = eos - bos;
            const long tok0 = (long)b * T + bos;
            const long VK = (long)V * K;
            const int nblk = (ntok + BWD_BLOCK - 1) / BWD_BLOCK;
            double *ck = (double *)malloc(sizeof(double) * VK * (size_t)(nblk + 1));
            double *Sb = (double *)malloc(sizeof(double) * VK * (BWD_BLOCK + 1));
            double *dS = (double *)malloc(sizeof(double) * VK);
            double *dD = (double *)malloc(sizeof(double) * VK);
            double *u = (double *)malloc(sizeof(double) * V);
            double *dr = (double *)malloc(sizeof(double) * V);
            for (int t = 0; t < ntok; ++t)
                for (int c = 0; c < K; ++c) {
                    dq[((tok0 + t) * HK + hk) * K + c] = 0.0;
                    dk[((tok0 + t) * HK + hk) * K + c] = 0.0;
                }
            for (int h = hk * grp; h < (hk + 1) * grp; ++h) {
                const float *kp = k + (tok0 * HK + hk) * K, *qp = q + (tok0 * HK + hk) * K;
                const float *vp = v + (tok0 * H + h) * V, *dop = dout + (tok0 * H + h) * V;
                const float *gp = g + tok0 * H + h, *bp = beta + tok0 * H + h;
                const long qs = (long)HK * K, vs = (long)H * V;
                /* checkpoints: the state before tokens 0, BWD_BLOCK, 2 BWD_BLOCK, ... */
                for (long i = 0; i < VK; ++i)
                    ck[i] = h0 ? (double)h0[((long)n * H + h) * VK + i] : 0.0;
                for (int bl = 0; bl < nblk; ++bl) {
                    memcpy(ck + VK * (bl + 1), ck + VK * bl, sizeof(double) * VK);
                    for (int t = bl * BWD_BLOCK; t < ntok && t < (bl + 1) * BWD_BLOCK; ++t)
                        gdn_token(ck + VK * (bl + 1), V, K, kp + t * qs, vp + t * vs,
                                  exp((double)gp[(long)t * H]), (double)bp[(long)t * H]);
                }
                for (long i = 0; i < VK; ++i)
                    dS[i] = dht ? (double)dht[((long)n * H + h) * VK + i] : 0.0;
                for (int bl = nblk - 1; bl >= 0; --bl) {
                    const int t0 = bl * BWD_BLOCK;
                    const int nt = (ntok - t0 < BWD_BLOCK) ? ntok - t0 : BWD_BLOCK;
                    /* Sb[i] = state before token t0 + i */
                    memcpy(Sb, ck + VK * bl, sizeof(double) * VK);
                    for (int i = 0; i < nt; ++i) {
                        memcpy(Sb + VK * (i + 1), Sb + VK * i, sizeof(double) * VK);
                        gdn_token(Sb + VK * (i + 1), V, K, kp + (t0 + i) * qs, vp + (t0 + i) * vs,
                                  exp((double)gp[(long)(t0 + i) * H]), (double)bp[(long)(t0 + i) * H]);
                    }
                    for (int i = nt - 1; i >= 0; --i) {
                        const int t = t0 + i;
                        const double *Sp = Sb + VK * i, *Sn = Sb + VK * (i + 1);
                        const float *kt = kp + t * qs, *qt = qp + t * qs, *vt = vp + t * vs, *dot = dop + t * vs;
                        const double gam = exp((double)gp[(long)t * H]), bt = (double)bp[(long)t * H];
                        double *dqt = dq + ((tok0 + t) * HK + hk) * K, *dkt = dk + ((tok0 + t) * HK + hk) * K;
                        /* o = scale S q */
                        for (int row = 0; row < V; ++row)
                            for (int c = 0; c < K; ++c) {
                                dS[(long)row * K + c] += scale * (double)dot[row] * (double)qt[c];
                                dqt[c] += scale * Sn[(long)row * K + c] * (double)dot[row];
                            }
                        /* S = D + r k^T with D = gamma S_prev, u = v - D k, r = beta u */
                        for (int row = 0; row < V; ++row) {
                            double dk_row = 0.0, acc = 0.0;
                            for (int c = 0; c < K; ++c) {
                                dk_row += gam * Sp[(long)row * K + c] * (double)kt[c];
                                acc += dS[(long)row * K + c] * (double)kt[c];
                            }
                            u[row] = (double)vt[row] - dk_row;
                            dr[row] = acc;
                        }
                        double db = 0.0;
                        for (int row = 0; row < V; ++row) {
                            db += dr[row] * u[row];
                            dv[(tok0 + t) * H * V + (long)h * V + row] = bt * dr[row];
                        }
                        dbeta[(tok0 + t) * H + h] = db;
                        for (int c = 0; c < K; ++c) {
                            double a1 = 0.0, a2 = 0.0;
                            for (int row = 0; row < V; ++row) {
                                a1 += dS[(long)row * K + c] * bt * u[row];          /* dS^T r */
                                a2 += gam * Sp[(long)row * K + c] * bt * dr[row];   /* D^T du */
                            }
                            dkt[c] += a1 - a2;
                        }
                        double dgam = 0.0;
                        for (int row = 0; row < V; ++row)
                            for (int c = 0; c < K; ++c) {
                                const long i2 = (long)row * K + c;
                                dD[i2] = dS[i2] - bt * dr[row] * (double)kt[c];
                                dgam += dD[i2] * Sp[i2];
                            }
                        dg[(tok0 + t) * H + h] = dgam * gam;
                        for (long i2 = 0; i2 < VK; ++i2)
                            dS[i2] = gam * dD[i2];
                    }
                }
                if (dh0)
                    memcpy(dh0 + ((long)n * H + h) * VK, dS, sizeof(double) * VK);
            }
            free(ck);
            free(Sb);
            free(dS);
            free(dD);
            free(u);
            free(dr);
        }
    }
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

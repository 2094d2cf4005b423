/*
 * sf.h -- C ABI of the chunk-parallel linear recurrence library for AMD
 * Instinct MI355X (gfx950).
 *
 * The library runs the forward pass of two linear recurrences on one GPU,
 * chunk by chunk, with hand-written HIP kernels:
 *
 *  - the Gated Delta Rule (attention-gym "Linear Attention" page, section
 *    "Gated Delta Rule"): per token, the state is decayed by exp(gate), the
 *    beta-scaled residual of the value against the decayed state read at the
 *    key is added as an outer product with the key, and the output is the
 *    scaled updated state read at the query;
 *  - scalar-gated linear attention (StateFlow, Section 2.1, Eq. (1), with the
 *    Mamba-2 scalar-identity transition; the SSD form of the Megatron-LM page
 *    "Mamba2 state-passing context parallelism"): S_t = exp(g_t) S_{t-1} +
 *    v_t k_t^T, o_t = scale * S_t q_t;
 *
 * plus the boundary-state passing that lets one long sequence be cut into
 * segments laid along the batch axis: every segment is an affine map of its
 * entry state (attention-gym "Context Parallelism"; the Megatron-LM page),
 * summarised independently, and the true entry states are recovered with an
 * exclusive scan over the summaries.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer to memory the caller owns
 *    (allocated with hipMalloc or by PyTorch). The library never allocates,
 *    frees or synchronises; it validates arguments on the host, enqueues its
 *    kernels on `stream` (a hipStream_t; NULL is the null stream) and returns.
 *  - Layouts are dense, row-major, token-major, with no padding:
 *      q, k  [B, T, HK, K]      v, out [B, T, H, V]
 *      g, beta [B, T, H] float32 (g is the natural-log decay, finite, <= 0)
 *      states [N, H, V, K] float32 (V-major: row v, column k)
 *    Value head h uses q/k head h / (H / HK); HK must divide H.
 *  - `dt` is the element type of q, k, v and out (SF_F32 or SF_BF16). Gates,
 *    beta, states and summaries are always float32; the recurrence is carried
 *    in float32.
 *  - cu_seqlens (optional, int32 [N + 1], device) packs N sequences into a
 *    batch-one stream: it starts at 0, never decreases and ends at or before
 *    T. Chunking restarts at every sequence start and a sequence's last chunk
 *    may be partial. An empty sequence returns its initial state as its final
 *    state. Output rows at or past cu_seqlens[N] are not written. These value
 *    constraints are the caller's responsibility and are not checked on the
 *    host (reading device memory would synchronise).
 *  - Inputs must not alias outputs.
 *  - Return value: SF_OK, or an error status with a message available from
 *    sf_last_error() (thread-local, valid until the next call on the same
 *    thread). Invalid shapes or pointers give SF_ERR_INVALID; shapes the
 *    kernels are not built for give SF_ERR_UNSUPPORTED (there is no fallback);
 *    a failed HIP launch gives SF_ERR_HIP. Nothing is enqueued when a call
 *    returns an error.
 *  - Sizes: every tensor must have fewer than 2^31 elements.
 */
#ifndef SF_H
#define SF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SF_OK = 0,
    SF_ERR_INVALID = 1,
    SF_ERR_UNSUPPORTED = 2,
    SF_ERR_HIP = 3,
    SF_ERR_WORKSPACE = 4
} sf_status;

typedef enum { SF_F32 = 0, SF_BF16 = 1 } sf_dtype;

typedef enum { SF_KIND_GDN = 0, SF_KIND_GLA = 1 } sf_kind;

/* Library version string, e.g. "sf 0.1.0 gfx950". */
const char *sf_version(void);

/* Message of the last non-OK status returned on this thread. */
const char *sf_last_error(void);

/*
 * Workspace bytes needed by sf_gdn_chunk_fwd for these sizes (packed != 0
 * when cu_seqlens is passed; then B must be 1). The workspace holds the
 * per-chunk factors of the chunk decomposition (StateFlow Section 2.2,
 * Eq. (2), "Pre"), one record per (64-token chunk, head): for bf16 the
 * unit-lower-triangular WY/UT solve factor scaled by beta (as MFMA fragments)
 * and the per-token decay coefficients; for float32 the solve factor, the
 * decay-masked query-key block and the coefficients. Packed inputs add the
 * device chunk table. Returns 0 for invalid sizes.
 */
size_t sf_gdn_chunk_fwd_workspace(sf_dtype dt, int B, int T, int H, int K, int V, int N,
                                  int packed);

/*
 * Gated Delta Rule chunk forward (attention-gym "Linear Attention", section
 * "Gated Delta Rule": chunk_gdn with a 64-token chunk).
 *   q, k   [B, T, HK, K] dt          v [B, T, H, V] dt
 *   g, beta [B, T, H] float32
 *   h0     [N, H, V, K] float32 initial states, or NULL for zeros
 *   cu_seqlens  int32 [N + 1] or NULL; without it N must equal B
 *   scale  query scale (the usual choice is 1 / sqrt(K), chosen by the caller)
 *   out    [B, T, H, V] dt           ht [N, H, V, K] float32 final states, or NULL
 *   q, k, v and out 16-byte aligned (SF_ERR_INVALID otherwise; the kernels move
 *          their rows in 16-byte pieces), as for every chunk-form entry point here
 *   workspace  at least sf_gdn_chunk_fwd_workspace(...) bytes, 256-byte aligned
 * Supported: K == V, K in {64, 128}.
 */
sf_status sf_gdn_chunk_fwd(sf_dtype dt, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *h0,
                           const int32_t *cu_seqlens, int N, int B, int T, int H, int HK,
                           int K, int V, float scale, void *out, float *ht,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes needed by sf_kda_chunk_fwd (packed != 0 when cu_seqlens is
 * passed): one float32 record per (64-token chunk, head) with the chunk's WY
 * factors W = T diag(beta) (Gamma o K) and U = T diag(beta) V, the decayed
 * query-key block P, the decayed queries and keys and the chunk's total decay,
 * and the device chunk table of packed inputs. 0 for invalid or unsupported
 * sizes. */
size_t sf_kda_chunk_fwd_workspace(sf_dtype dt, int B, int T, int H, int K, int V, int N,
                                  int packed);

/*
 * Kimi Delta Attention chunk forward (attention-gym "Linear Attention",
 * section "Kimi Delta Attention", chunk_kda with 64-token chunks): the delta
 * rule whose state decays key channel by key channel, with g the per-token,
 * per-channel natural-log decay (finite and <= 0, a caller responsibility),
 * as sf_kda_recurrent_fwd computes token by token.
 *   q, k, g [B, T, H, K] (g float32);  v [B, T, H, V];  beta [B, T, H] float32
 *   h0, cu_seqlens, N, scale, out, ht as sf_gdn_chunk_fwd (no grouped heads)
 *   workspace  at least sf_kda_chunk_fwd_workspace(...) bytes, 256-byte aligned
 * The within-chunk decay between two tokens is applied per pair and channel,
 * so the chunk form is exact for any nonpositive gate (no lower bound is
 * assumed). float32 arithmetic. Supported: (K, V) in {(128, 128), (128, 64),
 * (64, 64)}; others return SF_ERR_UNSUPPORTED.
 */
sf_status sf_kda_chunk_fwd(sf_dtype dt, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *h0,
                           const int32_t *cu_seqlens, int N, int B, int T, int H, int K, int V,
                           float scale, void *out, float *ht, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Workspace bytes needed by sf_gdn_chunk_bwd for these sizes (packed != 0 when
 * cu_seqlens is passed). It holds, in float32, one record per (64-token chunk,
 * head) with the chunk's solve factor T, its WY factor W = T diag(beta Gamma) K,
 * Qt = scale diag(Gamma) Q - P W and decay coefficients, every chunk's entry
 * state and the gradient of every chunk's exit state ([chunks, H, V, K] each),
 * and the device chunk table of packed inputs. Returns 0 for invalid sizes. */
size_t sf_gdn_chunk_bwd_workspace(sf_dtype dt, int B, int T, int H, int K, int V, int N,
                                  int packed);

/*
 * Gated Delta Rule chunk backward: the gradients of sf_gdn_chunk_fwd's loss
 * sum(dout * out) + sum(dht * ht) with respect to its inputs (the token rule of
 * attention-gym "Linear Attention", section "Gated Delta Rule", differentiated
 * through the chunk form of StateFlow Section 2.2, Eq. (2); the state gradient
 * runs from the last chunk back to the first as in its Eq. (6)-(7)).
 *   q, k, v, g, beta, h0, cu_seqlens, N, B, T, H, HK, K, V, scale
 *          as sf_gdn_chunk_fwd (h0 NULL: zero initial states)
 *   dout   [B, T, H, V] dt, the gradient of the output
 *   dht    [N, H, V, K] float32, the gradient of the final states, or NULL (zero)
 *   dq, dk [B, T, HK, K] dt;  dv [B, T, H, V] dt;  dg, dbeta [B, T, H] float32;
 *          q, k, v, dout, dq, dk and dv 16-byte aligned (SF_ERR_INVALID otherwise);
 *   dh0    [N, H, V, K] float32 or NULL (not written)
 *          Entries of tokens at or past cu_seqlens[N] are not written.
 *   workspace  at least sf_gdn_chunk_bwd_workspace(...) bytes, 256-byte aligned
 * All arithmetic is float32. Supported: HK == H, K and V in {64, 128}; others
 * return SF_ERR_UNSUPPORTED. Caller-owned device memory throughout; enqueued on
 * stream, no synchronisation.
 */
sf_status sf_gdn_chunk_bwd(sf_dtype dt, const void *q, const void *k, const void *v,
                           const float *g, const float *beta, const float *h0,
                           const void *dout, const float *dht, const int32_t *cu_seqlens,
                           int N, int B, int T, int H, int HK, int K, int V, float scale,
                           void *dq, void *dk, void *dv, float *dg, float *dbeta, float *dh0,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * sf_gdn_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results as sf_gdn_chunk_fwd without the workspace: the
 * workspace is a static device array of the library (sf_static_scratch_bytes()
 * bytes, 64 MiB; each GPU holds its own copy from the first call on it until
 * the process ends). Sizes whose workspace (sf_gdn_chunk_fwd_workspace) exceeds
 * it return SF_ERR_WORKSPACE with nothing enqueued. The entry point calls no
 * allocator. Every call on one GPU shares that GPU's array, so calls that
 * overlap on one GPU (other streams, other threads) race: the caller orders
 * them. Nothing in the array has to start at zero.
 */
sf_status sf_gdn_chunk_fwd_noalloc(sf_dtype dt, const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, const float *h0,
                                   const int32_t *cu_seqlens, int N, int B, int T, int H, int HK,
                                   int K, int V, float scale, void *out, float *ht, void *stream);

/* Bytes of the static device array behind sf_gdn_chunk_fwd_noalloc. */
size_t sf_static_scratch_bytes(void);

/*
 * Scalar-gated linear attention chunk forward (StateFlow Section 2.1, Eq. (1)
 * with F_t = exp(g_t) I; the Megatron-LM "Mamba2 state-passing context
 * parallelism" SSD core): S_t = exp(g_t) S_{t-1} + v_t k_t^T,
 * o_t = scale * S_t q_t. Same layouts as sf_gdn_chunk_fwd without beta.
 * chunk is 64 or 128 (64 only for SF_F32). Supported: K, V in {64, 128}.
 * Needs no workspace.
 */
sf_status sf_gla_chunk_fwd(sf_dtype dt, const void *q, const void *k, const void *v,
                           const float *g, const float *h0, const int32_t *cu_seqlens,
                           int N, int B, int T, int H, int HK, int K, int V, int chunk,
                           float scale, void *out, float *ht, void *stream);

/* Workspace bytes needed by sf_segment_summary (0 for SF_KIND_GLA). */
size_t sf_segment_summary_workspace(sf_kind kind, sf_dtype dt, int n_rows, int L_seg, int H,
                                    int K, int V, int chunk);

/*
 * Affine summary of each segment row (attention-gym "Context Parallelism":
 * a token range is the map S_out = S_in @ M + S_ext; its sub-section "cuDNN
 * local execution": S_ext is the exit state from a zero entry state and M
 * the exit state from the identity entry with the value term disabled;
 * Megatron-LM "Mamba2 state-passing context parallelism": for the scalar
 * gate, S_out = a_block * S_in + S_ext).
 *   k [n_rows, L_seg, HK, K] dt, v [n_rows, L_seg, H, V] dt, g and beta
 *   [n_rows, L_seg, H] float32 (beta NULL for SF_KIND_GLA). A long sequence
 *   [B, T, ...] is passed as its segment view [B * n_seg, T / n_seg, ...]
 *   (a reshape: row s = b * n_seg + j covers tokens [j L_seg, (j+1) L_seg)).
 *   M: SF_KIND_GDN  [n_rows, H, K, K] float32 transition
 *      SF_KIND_GLA  [n_rows, H] float32 a_block = exp(sum of the row's gates)
 *   S_ext [n_rows, H, V, K] float32.
 *   chunk: 64 for SF_KIND_GDN, 64 or 128 for SF_KIND_GLA; L_seg need not be
 *   a multiple of it (the last chunk may be partial).
 */
sf_status sf_segment_summary(sf_kind kind, sf_dtype dt, const void *k, const void *v,
                             const float *g, const float *beta, int n_rows, int L_seg, int H,
                             int HK, int K, int V, int chunk, float *M, float *S_ext,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Exclusive state scan over segment summaries (Megatron-LM "Mamba2
 * state-passing context parallelism": exclusive causal scan; attention-gym
 * "Context Parallelism": composition of range maps). For every batch row b
 * and segment j (row s = b * n_seg + j):
 *   S_in[b*n_seg]       = h0[b] (zeros if h0 is NULL)
 *   S_in[b*n_seg + j+1] = S_in[b*n_seg + j] @ M[s] + S_ext[s]     (SF_KIND_GDN)
 *                       = M[s] * S_in[b*n_seg + j] + S_ext[s]     (SF_KIND_GLA, M = a_block)
 *   S_final[b]          = the same step applied after the last segment
 *   M: [B*n_seg, H, K, K] (GDN) or [B*n_seg, H] (GLA); S_ext, S_in
 *   [B*n_seg, H, V, K]; h0, S_final [B, H, V, K] (S_final may be NULL).
 *   All float32. The products are carried in float32.
 */
sf_status sf_state_scan(sf_kind kind, const float *M, const float *S_ext, const float *h0,
                        int B, int n_seg, int H, int K, int V, float *S_in, float *S_final,
                        void *stream);

/* Workspace bytes needed by sf_gdn_segmented_fwd (0 for invalid sizes). */
size_t sf_gdn_segmented_fwd_workspace(sf_dtype dt, int B, int n_seg, int T, int H, int K, int V);

/*
 * Gated Delta Rule forward of B long sequences, each cut into n_seg contiguous
 * segments laid along the batch axis (Megatron-LM "Mamba2 state-passing
 * context parallelism": summarise every segment, recover the true entry
 * states with an exclusive scan, then finish each segment from its entry
 * state; attention-gym "Context Parallelism" for the delta rule's affine
 * range maps). The same result as sf_segment_summary, sf_state_scan and
 * sf_gdn_chunk_fwd on the segment view, with the chunk factors of every
 * segment formed once for both passes.
 *   q, k [B, T, HK, K] dt, v [B, T, H, V] dt, g and beta [B, T, H] float32;
 *   T a multiple of n_seg and T / n_seg a multiple of 64.
 *   h0 [B, H, V, K] float32 or NULL for zeros; out [B, T, H, V] dt;
 *   ht [B, H, V, K] float32 final states, or NULL.
 *   workspace at least sf_gdn_segmented_fwd_workspace(...) bytes, 256-byte
 *   aligned (it holds the factors, the summaries and the entry states).
 * Supported: K == V, K in {64, 128}.
 */
sf_status sf_gdn_segmented_fwd(sf_dtype dt, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *h0, int B,
                               int n_seg, int T, int H, int HK, int K, int V, float scale,
                               void *out, float *ht, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Gate transform kinds (attention-gym "Linear Attention", section "Gate Transforms"). */
typedef enum { SF_GATE_SOFTPLUS = 0, SF_GATE_BOUNDED = 1 } sf_gate_kind;

/*
 * sf_gdn_chunk_fwd with the gate transform fused into the gate load of its
 * Pre stage (attention-gym "Linear Attention", "Gate Transforms": no separate
 * elementwise kernel runs): g[b, t, h] is formed from raw_gate [B, T, H] in dt
 * as sf_gate_transform forms it for per-head gates (A_log [H], dt_bias [H],
 * float32; kind SF_GATE_SOFTPLUS or SF_GATE_BOUNDED with a finite
 * lower_bound <= 0), in float32. Every other argument, the workspace and the
 * results are those of sf_gdn_chunk_fwd.
 */
sf_status sf_gdn_chunk_fwd_raw_gate(sf_dtype dt, const void *q, const void *k, const void *v,
                                    const void *raw_gate, const float *A_log, const float *dt_bias,
                                    sf_gate_kind kind, float lower_bound, const float *beta,
                                    const float *h0, const int32_t *cu_seqlens, int N, int B, int T,
                                    int H, int HK, int K, int V, float scale, void *out, float *ht,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes needed by sf_paged_gdn_chunk_fwd (0 for invalid sizes). */
size_t sf_paged_gdn_chunk_fwd_workspace(sf_dtype dt, int B, int T, int H, int K, int V, int N,
                                        int packed);

/*
 * Delta-rule chunk forward on a paged state cache (attention-gym "Linear
 * Attention": the paged_chunk_gdn entry; inference prefill). As
 * sf_gdn_chunk_fwd, but sequence n starts from slot state_indices[n] of
 * state_pool (from zeros when has_initial_state is given and
 * has_initial_state[n] == 0) and its final state overwrites that slot,
 * even for an empty sequence; a non-positive index (or one >= num_slots)
 * gives zero output rows and leaves the pool alone. The pool layout is as for
 * sf_gdn_decode (pool_dt SF_F32 or SF_BF16; slot_stride elements between
 * slots, a multiple of 4 and >= H*V*K; 16-byte aligned). Two sequences naming
 * the same positive slot race. workspace: at least
 * sf_paged_gdn_chunk_fwd_workspace(...) bytes, 256-byte aligned (the chunk
 * path's records plus float32 entry and exit states). Supported shapes as
 * for sf_gdn_chunk_fwd.
 */
sf_status sf_paged_gdn_chunk_fwd(sf_dtype dt, const void *q, const void *k, const void *v,
                                 const float *g, const float *beta, const int32_t *cu_seqlens, int N,
                                 int B, int T, int H, int HK, int K, int V, float scale, void *out,
                                 void *state_pool, sf_dtype pool_dt, int num_slots,
                                 long long slot_stride, const int32_t *state_indices,
                                 const uint8_t *has_initial_state, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * Gate transform: raw gate projections to float32 natural-log decays
 * (attention-gym "Linear Attention", section "Gate Transforms"). For element e
 * of raw [rows, H, D] (D = 1: per-head gates [rows, H], dt_bias [H];
 * D > 1: per-channel gates, dt_bias [H, D]), j = e mod (H*D), h = j / D:
 *   SF_GATE_SOFTPLUS: out[e] = -exp(A_log[h]) * softplus(raw[e] + dt_bias[j])
 *   SF_GATE_BOUNDED:  out[e] = lower_bound * sigmoid(exp(A_log[h]) * (raw[e] + dt_bias[j]))
 * raw in dt (rows = the product of the leading dimensions, e.g. B*T), 8-byte
 * (bf16) or 16-byte (float32) aligned; A_log [H] and dt_bias float32; out
 * [rows, H, D] float32, 16-byte aligned. lower_bound is read by the bounded
 * kind only and must be finite and <= 0 there. Arithmetic is float32.
 */
sf_status sf_gate_transform(sf_dtype dt, const void *raw, const float *A_log, const float *dt_bias,
                            long long rows, int H, int D, sf_gate_kind kind, float lower_bound,
                            float *out, void *stream);

/*
 * Token-by-token Gated Delta Rule forward (attention-gym "Linear Attention":
 * the recurrent_gdn entry; the token rule of the section "Gated Delta Rule").
 * The same result as sf_gdn_chunk_fwd up to floating-point order, computed one
 * token after another with the state in registers: meant for decoding and for
 * short prefills (a few tokens per sequence), where the chunk path's per-chunk
 * factors do not pay. Measured on MI355X (H = 32, K = V = 128, bf16): faster
 * than sf_gdn_chunk_fwd at 16 tokens per sequence, 3x slower at 64 and 5x at
 * 1024; past a few dozen tokens call the chunk entry instead.
 *   q, k [B, T, HK, K] dt, v [B, T, H, V] dt, g and beta [B, T, H] float32
 *   (g the natural-log decay, beta the write gate, both used as given);
 *   cu_seqlens [N+1] (batch-one packed input) or NULL (then N == B);
 *   out [B, T, H, V] dt (rows at or past cu_seqlens[N] are not written).
 * State, one of two modes:
 *   - state_indices == NULL: h0 [N, H, V, K] float32 or NULL (zeros); ht
 *     [N, H, V, K] float32 or NULL; state_pool must be NULL;
 *   - state_indices [N] int32: sequence n starts from slot state_indices[n]
 *     of state_pool (zeros when has_initial_state[n] == 0) and its final
 *     state overwrites that slot, even for an empty sequence; an index <= 0 or
 *     >= num_slots gives zero output rows and no state access; h0 and ht must
 *     be NULL. The pool layout is as for sf_gdn_decode (pool_dt SF_F32 or
 *     SF_BF16, slot_stride elements between slots, each slot a dense
 *     [H, V, K] block, 16-byte aligned base); two sequences naming the same
 *     positive slot race.
 * K in {64, 128, 256}; V a positive multiple of 32; HK divides H.
 */
sf_status sf_gdn_recurrent_fwd(sf_dtype dt, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *h0,
                               const int32_t *cu_seqlens, int N, int B, int T, int H, int HK, int K,
                               int V, float scale, void *out, float *ht, void *state_pool,
                               sf_dtype pool_dt, int num_slots, long long slot_stride,
                               const int32_t *state_indices, const uint8_t *has_initial_state,
                               void *stream);

/*
 * Kimi Delta Attention, token by token (attention-gym "Linear Attention",
 * section "Kimi Delta Attention"), with a per-channel gate g_t in R^K:
 * decayed = S diag(exp(g_t)), r = beta_t (v_t - decayed k_t),
 * S = decayed + r k_t^T, o_t = scale S q_t.
 * Arguments, state modes and errors as sf_gdn_recurrent_fwd, except:
 *   q, k, g [B, T, H, K] (no grouped heads; g float32, 16-byte aligned).
 */
sf_status sf_kda_recurrent_fwd(sf_dtype dt, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *h0,
                               const int32_t *cu_seqlens, int N, int B, int T, int H, int K, int V,
                               float scale, void *out, float *ht, void *state_pool, sf_dtype pool_dt,
                               int num_slots, long long slot_stride, const int32_t *state_indices,
                               const uint8_t *has_initial_state, void *stream);

/*
 * One-token paged Gated Delta Rule decode (attention-gym "Linear Attention":
 * the recurrent_gdn_decode entry; section "Gate Transforms" for the gate).
 * For every sequence b < B and value head h < H, in float32:
 *   slot = state_indices[b]; a slot <= 0 (null row) or >= num_slots gives a
 *   zero output row and no state access;
 *   q, k = the row's query and key heads h / (H / HK), each L2-normalised as
 *   x / sqrt(|x|^2 + 1e-6); v = the row's value head h;
 *   g = -exp(A_log[h]) * softplus(raw_gate[b, h] + dt_bias[h]);
 *   beta = sigmoid(raw_beta[b, h]);
 *   S = state_pool[slot, h] (zeros when has_initial_state[b] == 0);
 *   S <- exp(g) S; r = beta (v - S k); S <- S + r k^T; o = scale S q;
 *   state_pool[slot, h] = S (rounded to pool_dt); out[b, h] = o (in dt).
 * Arguments (all device pointers):
 *   packed_qkv [B, 2*HK*K + H*V] dt, per row the HK query heads, the HK key
 *   heads, then the H value heads, each head's K or V elements contiguous;
 *   raw_gate, raw_beta [B, H] dt (the [1, B, H] projections);
 *   A_log, dt_bias [H] float32;
 *   state_pool: num_slots slots, slot s at state_pool + s * slot_stride
 *   elements of pool_dt (SF_F32 or SF_BF16), each a dense [H, V, K] block;
 *   slot_stride >= H*V*K and a multiple of 4; 16-byte aligned base;
 *   state_indices [B] int32; has_initial_state [B] uint8 or NULL (all set);
 *   out [B, H, V] dt, must not alias an input.
 * The pool is advanced in place: two rows naming the same positive slot race
 * (the caller keeps active slots unique). K in {64, 128, 256}; V a positive
 * multiple of 16; HK divides H.
 */
sf_status sf_gdn_decode(sf_dtype dt, const void *packed_qkv, const void *raw_gate,
                        const void *raw_beta, const float *A_log, const float *dt_bias,
                        void *state_pool, sf_dtype pool_dt, int num_slots, long long slot_stride,
                        const int32_t *state_indices, const uint8_t *has_initial_state, int B,
                        int H, int HK, int K, int V, float scale, void *out, void *stream);

/*
 * One-token paged Kimi Delta Attention decode (attention-gym "Linear
 * Attention": the recurrent_kda_decode entry). As sf_gdn_decode, except:
 *   packed_qkv [B, H*(2K + V)]: all H query heads, all H key heads, then the
 *   H value heads (no grouped heads);
 *   raw_gate [B, H, K] dt (the [1, B, H, K] projection) with dt_bias [H, K]
 *   float32 (16-byte aligned): a per-key-channel gate through the kind's
 *   transform (SF_GATE_BOUNDED, the entry's default with lower_bound -5, or
 *   SF_GATE_SOFTPLUS), each key column of the state decayed by its own factor
 *   exp(g) before the correction.
 */
sf_status sf_kda_decode(sf_dtype dt, const void *packed_qkv, const void *raw_gate,
                        const void *raw_beta, const float *A_log, const float *dt_bias,
                        sf_gate_kind kind, float lower_bound, void *state_pool, sf_dtype pool_dt,
                        int num_slots, long long slot_stride, const int32_t *state_indices,
                        const uint8_t *has_initial_state, int B, int H, int K, int V, float scale,
                        void *out, void *stream);

/*
 * Host-side argument checks for debugging. The entry points do not read device
 * memory, so the value constraints on cu_seqlens and state_indices are the
 * caller's (attention-gym "Linear Attention" states the same for its packed
 * offsets and slot indices). These two functions check a HOST copy of those
 * arrays and return SF_ERR_INVALID with a message naming the first violation;
 * they enqueue nothing and touch no device memory. The Python binding calls them
 * on every entry when the environment variable SF_VALIDATE is set to 1.
 *   sf_check_cu_seqlens: cu_seqlens_host [N + 1] starts at 0, never decreases and
 *     ends at or before T.
 *   sf_check_state_indices: state_indices_host [N]; every positive index is below
 *     num_slots and no positive index repeats (two sequences on one slot race).
 *     Non-positive indices (padding / null rows) are allowed.
 */
sf_status sf_check_cu_seqlens(const int32_t *cu_seqlens_host, int N, int T);
sf_status sf_check_state_indices(const int32_t *state_indices_host, int N, int num_slots);

/*
 * Kernel timing hook for measurement. While enabled, every kernel the
 * library enqueues is bracketed by a pair of HIP events recorded on the same
 * stream (events come from a pool created by sf_timing_enable, so no
 * allocation happens in the enqueue path). sf_timing_collect synchronises
 * on the recorded events and returns, per kernel name, the number of
 * launches and the summed elapsed milliseconds, then clears the records.
 *   max_pairs: capacity of the pool (enable), 0 disables and frees the pool.
 *   names/total_ms/launches: arrays of length max_kernels; returns the number
 *   of distinct kernels written, or -1 on error.
 */
sf_status sf_timing_enable(int max_pairs);
int sf_timing_collect(const char **names, double *total_ms, int *launches, int max_kernels);

#ifdef __cplusplus
}
#endif

#endif /* SF_H */

"""Recurrent (token-by-token) delta rule with a paged state pool, and the one-token paged decode,
float64 (test infrastructure; same rules as the rest of ``oracle/``: only tests, the smoke check
and the bench's CPU baseline may use it).

``gdn_recurrent_paged`` follows the ``recurrent_gdn`` entry of attention-gym "Linear Attention"
with ``state_indices`` (and serves the ``paged_chunk_gdn`` entry too: chunking changes only the
floating-point order of the same recurrence, and the slot rules are the same): every sequence starts from its slot of the pool (or from zero when its
``has_initial_state`` entry is false), runs the token rule over its tokens, and its final state
overwrites the slot; a non-positive index gives zero output and leaves the pool untouched. The
token recurrence itself is ``oracle.gdn_forward`` (oracle.c); this function only gathers and
scatters the slots around it.

``gdn_decode`` follows attention-gym "Linear Attention": the API entry of ``recurrent_gdn_decode`` (the
packed post-convolution [Q | K | V] row per token, grouped q/k heads, the paged state pool
advanced in place through slot indices, null slots, the fresh-slot mask) and the section
"Gate Transforms" (the softplus convention for the decay). The recurrence step is the token
rule of the section "Gated Delta Rule".

Readings where the pages leave a step open:
* L2 normalisation is x / sqrt(sum x^2 + eps) with eps = 1e-6 (the pages give no epsilon;
  some guard is needed for a zero row, and this one moves a unit-scale row by about 1e-6).
* raw gate and raw beta come in the same element type as the packed row.
* slot index 0 and negative indices are null rows: zero output, pool untouched.

Everything runs in float64 on the values as given (bf16 inputs arrive already rounded).
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6


def softplus(x):
    """log(1 + exp(x)) without overflow."""
    return np.logaddexp(0.0, x)


def decay_gate(raw_gate, A_log, dt_bias):
    """Natural-log decay of the softplus convention: -exp(A_log) * softplus(raw + dt_bias)."""
    return -np.exp(A_log) * softplus(raw_gate + dt_bias)


def write_gate(raw_beta):
    """Logistic sigmoid."""
    return 1.0 / (1.0 + np.exp(-raw_beta))


def l2_normalise(x, eps=L2_EPS):
    return x / np.sqrt(np.dot(x, x) + eps)


def gdn_decode(packed_qkv, raw_gate, raw_beta, A_log, dt_bias, state_pool, state_indices,
               has_initial_state=None, *, H, HK, K, V, scale=None):
    """One decode step for B sequences.

    packed_qkv [B, 2*HK*K + H*V]: per token the query heads, then the key heads, then the
    value heads, each head's row contiguous. raw_gate, raw_beta [B, H] (or [1, B, H]);
    A_log, dt_bias [H]; state_pool [num_slots, H, V, K]; state_indices [B] int;
    has_initial_state [B] bool or None (all True).

    Returns (out [B, H, V], pool [num_slots, H, V, K]), both float64; ``pool`` is a copy of
    ``state_pool`` with the selected slots advanced.
    """
    x = np.asarray(packed_qkv, dtype=np.float64)
    B = x.shape[0]
    assert x.shape[1] == 2 * HK * K + H * V and H % HK == 0
    rg = np.asarray(raw_gate, dtype=np.float64).reshape(B, H)
    rb = np.asarray(raw_beta, dtype=np.float64).reshape(B, H)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    pool = np.array(state_pool, dtype=np.float64, copy=True)
    idx = np.asarray(state_indices).astype(np.int64)
    init = np.ones(B, dtype=bool) if has_initial_state is None else np.asarray(has_initial_state, dtype=bool)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    out = np.zeros((B, H, V), dtype=np.float64)
    group = H // HK
    for b in range(B):
        slot = int(idx[b])
        if slot <= 0:
            continue
        for h in range(H):
            hk = h // group
            q = l2_normalise(x[b, hk * K:(hk + 1) * K])
            k = l2_normalise(x[b, HK * K + hk * K:HK * K + (hk + 1) * K])
            v = x[b, 2 * HK * K + h * V:2 * HK * K + (h + 1) * V]
            g = decay_gate(rg[b, h], A_log[h], dt_bias[h])
            beta = write_gate(rb[b, h])
            S = pool[slot, h].copy() if init[b] else np.zeros((V, K))
            # token rule: decay, delta correction against the decayed state, then read with q
            S = np.exp(g) * S
            r = beta * (v - S @ k)
            S = S + np.outer(r, k)
            out[b, h] = scale * (S @ q)
            pool[slot, h] = S
    return out, pool


def gdn_recurrent_paged(q, k, v, g, beta, state_pool, state_indices, has_initial_state=None,
                        cu_seqlens=None, scale=None):
    """q, k [B, T, HK, K]; v [B, T, H, V]; g, beta [B, T, H] (g the natural-log decay, beta the
    write gate, both as given); state_pool [num_slots, H, V, K]; state_indices [N] (N = B, or the
    number of packed sequences). Returns (out [B, T, H, V], pool), float64; rows of null sequences
    are zero, rows outside every sequence are NaN."""
    from . import gdn_forward
    q = np.asarray(q, dtype=np.float64)
    B, T, HK, K = q.shape
    H, V = np.shape(v)[2], np.shape(v)[3]
    idx = np.asarray(state_indices).astype(np.int64)
    N = idx.shape[0]
    init = np.ones(N, dtype=bool) if has_initial_state is None else np.asarray(has_initial_state, dtype=bool)
    pool = np.array(state_pool, dtype=np.float64, copy=True)
    h0 = np.zeros((N, H, V, K))
    for n in range(N):
        if idx[n] > 0 and init[n]:
            h0[n] = pool[idx[n]]
    out, ht = gdn_forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu_seqlens, scale=scale)
    cu = np.arange(B + 1) * T if cu_seqlens is None else np.asarray(cu_seqlens)
    for n in range(N):
        if idx[n] > 0:
            pool[idx[n]] = ht[n]
        else:  # a null sequence: zero output rows
            if cu_seqlens is None:
                out[n] = 0.0
            else:
                out[0, cu[n]:cu[n + 1]] = 0.0
    return out, pool


def gate_transform(raw, A_log, dt_bias, kind, lower_bound=None):
    """Raw gate projections to natural-log decays (attention-gym "Linear Attention", section "Gate
    Transforms"), float64. raw [..., H] with dt_bias [H] (per-head gates) or raw [..., H, D] with
    dt_bias [H, D] (per-channel gates); A_log [H].
      "softplus": -exp(A_log) * softplus(raw + dt_bias)
      "bounded":  lower_bound * sigmoid(exp(A_log) * (raw + dt_bias))"""
    raw = np.asarray(raw, dtype=np.float64)
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    H = A_log.shape[0]
    per_channel = dt_bias.ndim == 2
    assert raw.shape[-2 if per_channel else -1] == H and dt_bias.shape[0] == H
    amp = np.exp(A_log)[:, None] if per_channel else np.exp(A_log)
    x = raw + dt_bias
    if kind == "softplus":
        assert lower_bound is None
        return -amp * softplus(x)
    if kind == "bounded":
        assert lower_bound is not None and np.isfinite(lower_bound) and lower_bound <= 0
        return lower_bound * write_gate(amp * x)
    raise ValueError(kind)


def kda_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None):
    """Kimi Delta Attention, token by token (attention-gym "Linear Attention", section "Kimi Delta
    Attention"), float64, with a per-channel gate g_t in R^K: D = S diag(exp(g_t)),
    r = beta_t (v_t - D k_t), S = D + r k_t^T, o_t = scale S q_t.
    q, k, g [B, T, H, K]; v [B, T, H, V]; beta [B, T, H]; h0 [N, H, V, K] or None.
    Returns (out [B, T, H, V], ht [N, H, V, K]); rows outside every sequence are NaN."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, K = q.shape
    V = v.shape[3]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    if cu_seqlens is None:
        spans = [(n, 0, T) for n in range(B)]
    else:
        cu = np.asarray(cu_seqlens)
        assert B == 1
        spans = [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    N = len(spans)
    out = np.full((B, T, H, V), np.nan)
    ht = np.zeros((N, H, V, K))
    for n, (b, bos, eos) in enumerate(spans):
        S = np.zeros((H, V, K)) if h0 is None else np.array(h0[n], dtype=np.float64)
        for t in range(bos, eos):
            S = S * np.exp(g[b, t])[:, None, :]                      # channelwise decay of each key column
            r = beta[b, t][:, None] * (v[b, t] - np.einsum("hvk,hk->hv", S, k[b, t]))
            S = S + r[:, :, None] * k[b, t][:, None, :]
            out[b, t] = scale * np.einsum("hvk,hk->hv", S, q[b, t])
        ht[n] = S
    return out, ht


def kda_decode(packed_qkv, raw_gate, raw_beta, A_log, dt_bias, state_pool, state_indices,
               has_initial_state=None, *, H, K, V, kind="bounded", lower_bound=-5.0, scale=None):
    """One-token paged KDA decode (attention-gym "Linear Attention", the recurrent_kda_decode entry):
    packed_qkv [B, H (2K + V)] (all query heads, all key heads, all value heads); raw_gate [B, H, K]
    (or [1, B, H, K]) through gate_transform with dt_bias [H, K] (per-channel); raw_beta [B, H] through
    the sigmoid; q and k L2-normalised; then the KDA token rule on the slot's state. Slot rules as
    gdn_decode. Returns (out [B, H, V], pool), float64."""
    x = np.asarray(packed_qkv, dtype=np.float64)
    B = x.shape[0]
    assert x.shape[1] == H * (2 * K + V)
    rg = np.asarray(raw_gate, dtype=np.float64).reshape(B, H, K)
    rb = np.asarray(raw_beta, dtype=np.float64).reshape(B, H)
    gate = gate_transform(rg, A_log, dt_bias, kind, lower_bound if kind == "bounded" else None)  # [B, H, K]
    pool = np.array(state_pool, dtype=np.float64, copy=True)
    idx = np.asarray(state_indices).astype(np.int64)
    init = np.ones(B, dtype=bool) if has_initial_state is None else np.asarray(has_initial_state, dtype=bool)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    out = np.zeros((B, H, V))
    for b in range(B):
        slot = int(idx[b])
        if slot <= 0:
            continue
        for h in range(H):
            q = l2_normalise(x[b, h * K:(h + 1) * K])
            k = l2_normalise(x[b, H * K + h * K:H * K + (h + 1) * K])
            v = x[b, 2 * H * K + h * V:2 * H * K + (h + 1) * V]
            S = pool[slot, h].copy() if init[b] else np.zeros((V, K))
            S = S * np.exp(gate[b, h])[None, :]      # channelwise decay of the key columns
            r = write_gate(rb[b, h]) * (v - S @ k)
            S = S + np.outer(r, k)
            out[b, h] = scale * (S @ q)
            pool[slot, h] = S
    return out, pool


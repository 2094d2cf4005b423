"""Pins of the float64 oracle against facts that do not reuse its code.

Every check below would fail for a plausible slip in oracle.c (a dropped decay,
the residual taken against the undecayed state, the output read before the
update, a transposed summary, an inclusive instead of exclusive scan, a wrong
q/k group, a chunk that does not restart at a sequence start):

* general-recurrence form: StateFlow Section 2.1 Eq. (1), S_t = S_{t-1} F_t + u_t k_t^T,
  with the Gated Delta Rule's scalar-plus-low-rank transition
  F_t = exp(g_t) (I - beta_t k_t k_t^T), u_t = beta_t v_t, computed with dense
  numpy matrix products (attention-gym "Linear Attention", Gated Delta Rule);
* closed forms: beta = 0 gives pure decay; g = 0, beta = 1 with orthonormal keys
  overwrites the value stored under each key; the unit-key invariant
  S_t k_t = (1 - beta_t) exp(g_t) S_{t-1} k_t + beta_t v_t;
* scalar gate: the masked quadratic form (D o Q K^T) V of the SSD dual and, at
  g = 0, causal linear attention tril(Q K^T) V;
* summaries (attention-gym "Context Parallelism"; Megatron-LM "Mamba2
  state-passing context parallelism"): M equals the ordered product of the
  transitions, affinity in the entry state, identity for an empty range,
  composition of two ranges, segmented run (summary + exclusive scan) equals
  the unsegmented run;
* packing: a packed stream equals separate runs, an empty sequence passes its
  state through, rows past the terminal offset are never written;
* chunk algebra (StateFlow Eq. (2)): the chunked form equals the recurrence.
"""
import numpy as np
import pytest

import workloads as wl

RNG = np.random.default_rng(20261202)


def rand_gdn(B=1, T=9, H=2, HK=None, K=5, V=3, h0=True, unit=True, seed=0, gate_shift=0.0):
    rng = np.random.default_rng(seed)
    HK = HK or H
    q = rng.standard_normal((B, T, HK, K))
    k = rng.standard_normal((B, T, HK, K))
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, V))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H)) + gate_shift))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = rng.standard_normal((B, H, V, K)) * 0.5 if h0 else None
    f32 = lambda x: None if x is None else x.astype(np.float32)
    return [f32(x) for x in (q, k, v, g, beta, s0)]


# ---------------------------------------------------------------------------
# Gated Delta Rule, token rule
# ---------------------------------------------------------------------------

def eq1_reference(q, k, v, g, beta, h0, scale):
    """Dense Eq. (1) form with F_t = exp(g_t)(I - beta_t k k^T), u_t = beta_t v_t."""
    B, T, HK, K = q.shape
    H, V = v.shape[2:]
    grp = H // HK
    out = np.zeros((B, T, H, V))
    ht = np.zeros((B, H, V, K))
    I = np.eye(K)
    for b in range(B):
        for h in range(H):
            S = np.zeros((V, K)) if h0 is None else h0[b, h].astype(np.float64)
            for t in range(T):
                kt = k[b, t, h // grp].astype(np.float64)
                F = np.exp(float(g[b, t, h])) * (I - float(beta[b, t, h]) * np.outer(kt, kt))
                S = S @ F + float(beta[b, t, h]) * np.outer(v[b, t, h], kt)
                out[b, t, h] = scale * S @ q[b, t, h // grp]
            ht[b, h] = S
    return out, ht


@pytest.mark.parametrize("HK", [2, 1])
def test_gdn_matches_general_recurrence(oracle, HK):
    q, k, v, g, beta, h0 = rand_gdn(B=2, T=11, H=2, HK=HK, K=6, V=4, seed=1)
    o, ht = oracle.gdn_forward(q, k, v, g, beta, h0, scale=0.7)
    o2, ht2 = eq1_reference(q, k, v, g, beta, h0, 0.7)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ht, ht2, rtol=0, atol=1e-12)


def test_gdn_default_scale(oracle):
    q, k, v, g, beta, h0 = rand_gdn(T=4, K=9, V=2, seed=2)
    o, _ = oracle.gdn_forward(q, k, v, g, beta, h0)
    o2, _ = oracle.gdn_forward(q, k, v, g, beta, h0, scale=1.0 / 3.0)
    np.testing.assert_array_equal(o, o2)


def test_gdn_beta_zero_is_pure_decay(oracle):
    q, k, v, g, beta, h0 = rand_gdn(T=13, K=5, V=3, seed=3)
    beta[:] = 0.0
    o, ht = oracle.gdn_forward(q, k, v, g, beta, h0, scale=1.0)
    G = np.cumsum(g.astype(np.float64), axis=1)            # [B, T, H]
    for h in range(g.shape[2]):
        np.testing.assert_allclose(ht[0, h], np.exp(G[0, -1, h]) * h0[0, h], rtol=1e-13, atol=0)
        for t in range(g.shape[1]):
            want = np.exp(G[0, t, h]) * h0[0, h].astype(np.float64) @ q[0, t, h]
            np.testing.assert_allclose(o[0, t, h], want, rtol=1e-12, atol=1e-14)


def test_gdn_overwrite_with_orthonormal_keys(oracle):
    K, V, T = 8, 5, 20
    rng = np.random.default_rng(4)
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    idx = rng.integers(0, 5, size=T)                       # keys drawn with repeats from 5 rows
    k = Qm[idx].reshape(1, T, 1, K).astype(np.float32)
    q = k.copy()                                           # read the key just written
    v = rng.standard_normal((1, T, 1, V)).astype(np.float32)
    g = np.zeros((1, T, 1), np.float32)
    beta = np.ones((1, T, 1), np.float32)
    h0 = rng.standard_normal((1, 1, V, K)).astype(np.float32)
    o, ht = oracle.gdn_forward(q, k, v, g, beta, h0, scale=1.0)
    kk = k[0, :, 0].astype(np.float64)
    # reading the key just written returns the value just written
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], rtol=0, atol=1e-5)
    used = sorted(set(idx.tolist()))
    last = {i: max(t for t in range(T) if idx[t] == i) for i in used}
    P = sum(np.outer(Qm[i], Qm[i]) for i in used)
    want = h0[0, 0].astype(np.float64) @ (np.eye(K) - P) + sum(
        np.outer(v[0, last[i], 0], Qm[i]) for i in used)
    np.testing.assert_allclose(ht[0, 0], want, rtol=0, atol=1e-5)


def test_gdn_unit_key_invariant(oracle):
    q, k, v, g, beta, h0 = rand_gdn(T=10, K=7, V=4, H=1, seed=5)
    prev = h0[0, 0].astype(np.float64)
    for t in range(1, 11):
        _, ht = oracle.gdn_forward(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], h0)
        kt = k[0, t - 1, 0].astype(np.float64)
        kt_n = kt / np.linalg.norm(kt)                      # float32 unit rows are unit to ~1e-7
        lhs = ht[0, 0] @ kt
        b, gam = float(beta[0, t - 1, 0]), np.exp(float(g[0, t - 1, 0]))
        rhs = (1 - b * (kt @ kt)) * gam * prev @ kt + b * (kt @ kt) * v[0, t - 1, 0]
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)
        assert abs(np.linalg.norm(kt_n) - 1) < 1e-12
        prev = ht[0, 0]


# ---------------------------------------------------------------------------
# Scalar-gated linear attention
# ---------------------------------------------------------------------------

def rand_gla(B=1, T=12, H=4, HK=2, K=6, V=3, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, HK, K)).astype(np.float32)
    k = rng.standard_normal((B, T, HK, K)).astype(np.float32)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((B, T, H))))).astype(np.float32)
    return q, k, v, g


def test_gla_equals_masked_quadratic_form(oracle):
    q, k, v, g = rand_gla(B=2, seed=6)
    o, _ = oracle.gla_forward(q, k, v, g, scale=0.5)
    grp = v.shape[2] // q.shape[2]
    for b in range(2):
        for h in range(v.shape[2]):
            G = np.cumsum(g[b, :, h].astype(np.float64))
            D = np.tril(np.exp(G[:, None] - G[None, :]))
            Qh, Kh = q[b, :, h // grp].astype(np.float64), k[b, :, h // grp].astype(np.float64)
            want = 0.5 * (D * (Qh @ Kh.T)) @ v[b, :, h]
            np.testing.assert_allclose(o[b, :, h], want, rtol=1e-12, atol=1e-12)


def test_gla_zero_gate_is_causal_linear_attention(oracle):
    q, k, v, g = rand_gla(seed=7, HK=4)
    g[:] = 0
    o, ht = oracle.gla_forward(q, k, v, g)
    for h in range(4):
        Qh, Kh, Vh = (x[0, :, h].astype(np.float64) for x in (q, k, v))
        np.testing.assert_allclose(o[0, :, h], np.tril(Qh @ Kh.T) @ Vh, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(ht[0, h], Vh.T @ Kh, rtol=1e-12, atol=1e-12)


def test_gla_with_initial_state_closed_form(oracle):
    q, k, v, g = rand_gla(seed=8, HK=1, H=2)
    h0 = np.random.default_rng(9).standard_normal((1, 2, 3, 6)).astype(np.float32)
    o, ht = oracle.gla_forward(q, k, v, g, h0=h0)
    for h in range(2):
        G = np.cumsum(g[0, :, h].astype(np.float64))
        Qh, Kh, Vh = q[0, :, 0].astype(np.float64), k[0, :, 0].astype(np.float64), v[0, :, h]
        D = np.tril(np.exp(G[:, None] - G[None, :]))
        want = np.exp(G)[:, None] * (Qh @ h0[0, h].astype(np.float64).T) + (D * (Qh @ Kh.T)) @ Vh
        np.testing.assert_allclose(o[0, :, h], want, rtol=1e-12, atol=1e-12)
        Sf = np.exp(G[-1]) * h0[0, h] + (np.exp(G[-1] - G)[:, None] * Vh).T @ Kh
        np.testing.assert_allclose(ht[0, h], Sf, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# Summaries and the exclusive scan
# ---------------------------------------------------------------------------

def test_gdn_summary_is_product_of_transitions(oracle):
    q, k, v, g, beta, _ = rand_gdn(T=9, H=2, HK=1, K=5, V=3, seed=10)
    M, S_ext = oracle.gdn_summary(k, v, g, beta)
    for h in range(2):
        P = np.eye(5)
        E = np.zeros((3, 5))
        for t in range(9):
            kt = k[0, t, 0].astype(np.float64)
            F = np.exp(float(g[0, t, h])) * (np.eye(5) - float(beta[0, t, h]) * np.outer(kt, kt))
            P = P @ F
            E = E @ F + float(beta[0, t, h]) * np.outer(v[0, t, h], kt)
        np.testing.assert_allclose(M[0, h], P, rtol=0, atol=1e-13)
        np.testing.assert_allclose(S_ext[0, h], E, rtol=0, atol=1e-13)


@pytest.mark.parametrize("kind", ["gdn", "gla"])
def test_summary_is_affine_in_entry_state(oracle, kind):
    q, k, v, g, beta, h0 = rand_gdn(B=2, T=17, H=2, K=6, V=4, seed=11)
    if kind == "gdn":
        _, ht = oracle.gdn_forward(q, k, v, g, beta, h0)
        M, E = oracle.gdn_summary(k, v, g, beta)
        want = np.einsum("bhvk,bhkj->bhvj", h0.astype(np.float64), M) + E
    else:
        _, ht = oracle.gla_forward(q, k, v, g, h0=h0)
        a, E = oracle.gla_summary(k, v, g)
        want = a[:, :, None, None] * h0 + E
    np.testing.assert_allclose(ht, want, rtol=0, atol=1e-12)


def test_summary_of_empty_range_is_identity(oracle):
    q, k, v, g, beta, _ = rand_gdn(T=8, H=2, K=4, V=3, seed=12)
    cu = np.array([0, 3, 3, 8], np.int32)
    M, E = oracle.gdn_summary(k, v, g, beta, cu_seqlens=cu)
    np.testing.assert_array_equal(M[1], np.broadcast_to(np.eye(4), (2, 4, 4)))
    np.testing.assert_array_equal(E[1], 0)
    a, E2 = oracle.gla_summary(k, v, g, cu_seqlens=cu)
    np.testing.assert_array_equal(a[1], 1.0)
    np.testing.assert_array_equal(E2[1], 0)


def test_summary_composition(oracle):
    q, k, v, g, beta, _ = rand_gdn(T=14, H=2, K=5, V=3, seed=13)
    cu = np.array([0, 6, 14], np.int32)
    M, E = oracle.gdn_summary(k, v, g, beta, cu_seqlens=cu)
    Mw, Ew = oracle.gdn_summary(k, v, g, beta)
    np.testing.assert_allclose(Mw[0], np.einsum("hij,hjk->hik", M[0], M[1]), atol=1e-13, rtol=0)
    np.testing.assert_allclose(Ew[0], np.einsum("hvk,hkj->hvj", E[0], M[1]) + E[1], atol=1e-13, rtol=0)


def _segment_view(x, n_seg):
    B, T = x.shape[:2]
    return x.reshape(B * n_seg, T // n_seg, *x.shape[2:])


@pytest.mark.parametrize("kind", ["gdn", "gla"])
def test_segmented_equals_unsegmented(oracle, kind):
    B, T, n_seg = 2, 48, 4
    q, k, v, g, beta, h0 = rand_gdn(B=B, T=T, H=2, K=6, V=4, seed=14, gate_shift=-3.0)
    seg = lambda x: _segment_view(x, n_seg)
    if kind == "gdn":
        o, ht = oracle.gdn_forward(q, k, v, g, beta, h0)
        M, E = oracle.gdn_summary(seg(k), seg(v), seg(g), seg(beta))
    else:
        o, ht = oracle.gla_forward(q, k, v, g, h0=h0)
        M, E = oracle.gla_summary(seg(k), seg(v), seg(g))
    S_in, S_final = oracle.state_scan(kind, M, E, h0, B=B, n_seg=n_seg)
    # exclusive: the first segment of each row starts from h0 itself
    np.testing.assert_array_equal(S_in[0::n_seg], h0.astype(np.float64))
    # the scan is exercised: transitions are far from zero
    assert (np.abs(M).max() if kind == "gdn" else M.min()) > 0.1
    if kind == "gdn":
        os_, hs = oracle.gdn_forward(seg(q), seg(k), seg(v), seg(g), seg(beta), S_in.astype(np.float32))
        # S_in is rounded to float32 above only to pass it as an entry state; compare loosely there
        tol = 1e-5
    else:
        os_, hs = oracle.gla_forward(seg(q), seg(k), seg(v), seg(g), h0=S_in.astype(np.float32))
        tol = 1e-5
    np.testing.assert_allclose(os_.reshape(o.shape), o, rtol=0, atol=tol)
    np.testing.assert_allclose(S_final, ht, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hs[n_seg - 1::n_seg], ht, rtol=0, atol=tol)


def test_scan_matches_direct_summary_of_whole_row(oracle):
    """S_final from the scan of per-segment summaries equals h0 @ M_whole + E_whole."""
    B, T, n_seg = 1, 40, 5
    q, k, v, g, beta, h0 = rand_gdn(B=B, T=T, H=1, K=4, V=3, seed=15, gate_shift=-4.0)
    M, E = oracle.gdn_summary(_segment_view(k, n_seg), _segment_view(v, n_seg),
                              _segment_view(g, n_seg), _segment_view(beta, n_seg))
    Mw, Ew = oracle.gdn_summary(k, v, g, beta)
    _, S_final = oracle.state_scan("gdn", M, E, h0, B=B, n_seg=n_seg)
    np.testing.assert_allclose(S_final[0, 0], h0[0, 0] @ Mw[0, 0] + Ew[0, 0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Packing, grouped heads, chunk algebra
# ---------------------------------------------------------------------------

def test_packed_equals_separate_runs(oracle):
    lens = [5, 0, 9, 1, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1]) + 3                                      # capacity past the terminal offset
    q, k, v, g, beta, _ = rand_gdn(T=T, H=2, K=5, V=3, seed=16)
    h0 = np.random.default_rng(17).standard_normal((len(lens), 2, 3, 5)).astype(np.float32)
    o, ht = oracle.gdn_forward(q, k, v, g, beta, h0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        s = slice(cu[n], cu[n + 1])
        o1, h1 = oracle.gdn_forward(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], h0[n:n + 1])
        np.testing.assert_array_equal(o[:, s], o1)
        np.testing.assert_array_equal(ht[n], h1[0])
    np.testing.assert_array_equal(ht[1], h0[1].astype(np.float64))  # empty sequence passes through
    assert np.isnan(o[0, cu[-1]:]).all()                     # rows past the terminal offset untouched


def test_grouped_heads_equal_expanded_heads(oracle):
    q, k, v, g, beta, h0 = rand_gdn(T=10, H=4, HK=2, K=5, V=3, seed=18)
    o, ht = oracle.gdn_forward(q, k, v, g, beta, h0)
    qe, ke = np.repeat(q, 2, axis=2), np.repeat(k, 2, axis=2)
    o2, ht2 = oracle.gdn_forward(qe, ke, v, g, beta, h0)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(ht, ht2)


@pytest.mark.parametrize("T", [1, 5, 16, 17, 40])
@pytest.mark.parametrize("kind", ["gdn", "gla"])
def test_chunked_equals_recurrent(oracle, kind, T):
    q, k, v, g, beta, h0 = rand_gdn(B=2, T=T, H=2, HK=1, K=6, V=5, seed=19 + T)
    if kind == "gdn":
        o, ht = oracle.gdn_forward(q, k, v, g, beta, h0)
    else:
        o, ht = oracle.gla_forward(q, k, v, g, h0=h0, scale=1.0 / np.sqrt(6))
    oc, hc = oracle.chunked_forward(kind, q, k, v, g, beta, h0, chunk=16, scale=1.0 / np.sqrt(6))
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hc, ht, rtol=0, atol=1e-12)


def test_chunked_restarts_at_sequence_starts(oracle):
    lens = [21, 0, 16, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta, _ = rand_gdn(T=int(cu[-1]), H=2, K=4, V=3, seed=30, gate_shift=-2.0)
    o, ht = oracle.gdn_forward(q, k, v, g, beta, cu_seqlens=cu)
    oc, hc = oracle.chunked_forward("gdn", q, k, v, g, beta, cu_seqlens=cu, chunk=8)
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hc, ht, rtol=0, atol=1e-12)


def test_chunked_survives_underflowing_gates(oracle):
    """Sum of gates within one chunk far below the float64 exponent range of exp (-800):
    the chunk form must only use exp of nonpositive gate differences."""
    q, k, v, g, beta, h0 = rand_gdn(T=32, H=1, K=4, V=3, seed=31)
    g[:] = -40.0
    o, ht = oracle.gdn_forward(q, k, v, g, beta, h0)
    oc, hc = oracle.chunked_forward("gdn", q, k, v, g, beta, h0, chunk=32)
    assert np.isfinite(oc).all()
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hc, ht, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Workload generator (host logic)
# ---------------------------------------------------------------------------

def test_varlen_lengths_recipe():
    rng = np.random.default_rng(wl.SEEDS["varlen_gdn"])
    lens = wl.varlen_lengths(rng, 32768)
    assert len(lens) == 9 and lens.sum() == 32768
    assert (lens == 0).sum() == 1
    nz = lens[lens > 0]
    assert (nz % 64 != 0).sum() >= 3 and nz.min() < 64
    again = wl.varlen_lengths(np.random.default_rng(wl.SEEDS["varlen_gdn"]), 32768)
    np.testing.assert_array_equal(lens, again)


def test_tiny_config_is_seeded_and_shaped():
    a, b = wl.tiny_gdn(), wl.tiny_gdn()
    assert a.q.shape == (1, 256, 2, 64) and a.q.dtype.is_floating_point
    for x, y in zip((a.q, a.k, a.v, a.g, a.beta), (b.q, b.k, b.v, b.g, b.beta)):
        assert (x == y).all()
    assert float(a.g.max()) <= 0.0 and 0.0 < float(a.beta.min()) and float(a.beta.max()) < 1.0
    np.testing.assert_allclose(np.linalg.norm(wl.to_f32(a.k), axis=-1), 1.0, atol=1e-5)


# ---------------------------------------------------------------------------
# Float32 build (CPU throughput baseline only)
# ---------------------------------------------------------------------------

def test_float32_build_matches_general_recurrence(oracle):
    """The float32 token loops against the dense Eq. (1) form in float64 (delta rule) and the
    masked quadratic SSD form (scalar gate), at float32 rounding: a slip in those loops (a
    dropped decay, the output read before the update) fails here even though they are never a
    parity reference."""
    lens = [40, 0, 17]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, g, beta, _ = rand_gdn(T=int(cu[-1]), H=2, K=8, V=6, seed=41, gate_shift=-1.0)
    h0 = (np.random.default_rng(3).standard_normal((3, 2, 6, 8)) * 0.3).astype(np.float32)
    o32, h32 = oracle.forward_f32("gdn", q, k, v, g, beta, h0, cu_seqlens=cu, scale=0.4)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        sl = lambda x: x[:, a:b]
        ro, rh = eq1_reference(sl(q), sl(k), sl(v), sl(g), sl(beta), h0[n:n + 1], 0.4)
        np.testing.assert_allclose(o32[:, a:b], ro, rtol=0, atol=2e-5)
        np.testing.assert_allclose(h32[n], rh[0], rtol=0, atol=2e-5)
    # scalar gate, zero initial state: O = (D o Q K^T) V with D_ti = exp(G_t - G_i), i <= t
    T = 37
    rng = np.random.default_rng(5)
    q2, k2, v2 = (rng.standard_normal((1, T, 1, 4)).astype(np.float32) for _ in range(3))
    g2 = -np.abs(rng.standard_normal((1, T, 1))).astype(np.float32) * 0.3
    o2, _ = oracle.forward_f32("gla", q2, k2, v2, g2, scale=1.0)
    G = np.cumsum(g2[0, :, 0].astype(np.float64))
    D = np.tril(np.exp(G[:, None] - G[None, :]))
    ref = (D * (q2[0, :, 0].astype(np.float64) @ k2[0, :, 0].T.astype(np.float64))) @ v2[0, :, 0]
    np.testing.assert_allclose(o2[0, :, 0], ref, rtol=0, atol=1e-4 * max(1.0, np.abs(ref).max()))

"""Pins of the float64 decode oracle (oracle/decode.py) against facts that do not reuse its code.

Each check would fail for a plausible slip in it: the decay with the wrong sign or without
exp(A_log), softplus or sigmoid swapped, a missing L2 normalisation, the residual taken against
the undecayed state, the output read before the update, the wrong q/k head for a value head,
sections of the packed row in the wrong order, a null slot written, a fresh slot read.

* closed forms of the gate transforms (attention-gym "Linear Attention", "Gate Transforms"):
  softplus(0) = ln 2, so A_log = ln 3 with a zero pre-activation decays by exactly 2^-3;
  sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4;
* single steps with a closed-form result: pure decay (beta -> 0) and a write into a fresh slot
  with q = k along one axis;
* invariance of the output under positive rescaling of q and k (the normalisation);
* T decode steps against the token-by-token float64 recurrence of oracle.c, which has pins of
  its own (tests/test_oracle.py), with grouped heads and a permuted set of slots.

The paged recurrent form (``gdn_recurrent_paged``: slot gather, ``gdn_forward``, slot scatter)
is pinned against the decode oracle run token by token (its q, k and gates prepared with the
decode module's own pinned helpers), and for null, fresh and empty sequences in a packed stream.
"""
import math

import numpy as np

import oracle
from oracle import decode as dec

H, HK, K, V = 4, 2, 8, 6


def packed(q, k, v):
    """[B, HK, K], [B, HK, K], [B, H, V] -> [B, 2 HK K + H V]."""
    B = q.shape[0]
    return np.concatenate([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)], axis=1)


def test_gate_transform_closed_forms():
    assert math.isclose(dec.decay_gate(0.0, 0.0, 0.0), -math.log(2.0), rel_tol=1e-15)
    assert math.isclose(dec.decay_gate(0.0, math.log(3.0), 0.0), -3 * math.log(2.0), rel_tol=1e-15)
    # the bias adds to the raw projection before softplus: softplus(ln 3 - ln 3 + 0) = ln 2
    assert math.isclose(dec.decay_gate(math.log(3.0), 0.0, -math.log(3.0)), -math.log(2.0), rel_tol=1e-15)
    # softplus(ln(e - 1)) = 1
    assert math.isclose(dec.softplus(math.log(math.e - 1.0)), 1.0, rel_tol=1e-15)
    assert math.isclose(dec.softplus(60.0), 60.0, rel_tol=1e-15)
    assert dec.softplus(-60.0) > 0.0
    assert dec.write_gate(0.0) == 0.5
    assert math.isclose(dec.write_gate(math.log(3.0)), 0.75, rel_tol=1e-15)


def _single(rng, B=2):
    q = rng.standard_normal((B, HK, K))
    k = rng.standard_normal((B, HK, K))
    v = rng.standard_normal((B, H, V))
    return q, k, v


def test_pure_decay_step():
    """beta -> 0: the state decays by exp(g) = 1/8 and the output reads the decayed state."""
    rng = np.random.default_rng(1)
    B, j = 2, 3
    q = np.zeros((B, HK, K))
    q[..., j] = 5.0                       # q-hat = e_j up to the normalisation guard
    _, k, v = _single(rng, B)
    pool = rng.standard_normal((4, H, V, K))
    idx = np.array([3, 1])
    out, new = oracle.gdn_decode(packed(q, k, v), np.zeros((B, H)), np.full((B, H), -80.0),
                                 np.full(H, math.log(3.0)), np.zeros(H), pool, idx,
                                 H=H, HK=HK, K=K, V=V, scale=0.5)
    shrink = 5.0 / math.sqrt(25.0 + dec.L2_EPS)
    for b in range(B):
        np.testing.assert_allclose(new[idx[b]], pool[idx[b]] / 8.0, rtol=1e-12, atol=1e-30)
        np.testing.assert_allclose(out[b], 0.5 * shrink * pool[idx[b]][:, :, j] / 8.0, rtol=1e-12)
    # untouched slots stay bit-identical
    for s in (0, 2):
        assert np.array_equal(new[s], pool[s])


def test_fresh_slot_write():
    """Fresh slot (garbage ignored), beta = 1/2, q = k = c e_j: S = v k-hat^T / 2, o = scale v/2 (k-hat.q-hat)."""
    rng = np.random.default_rng(2)
    B, j = 1, 5
    q = np.zeros((B, HK, K))
    q[..., j] = 3.0
    k = q.copy()
    v = rng.standard_normal((B, H, V))
    pool = np.full((2, H, V, K), np.nan)
    out, new = oracle.gdn_decode(packed(q, k, v), rng.standard_normal((B, H)), np.zeros((B, H)),
                                 rng.standard_normal(H), rng.standard_normal(H), pool, np.array([1]),
                                 np.array([False]), H=H, HK=HK, K=K, V=V, scale=0.25)
    c = 3.0 / math.sqrt(9.0 + dec.L2_EPS)
    expect_S = np.zeros((H, V, K))
    expect_S[:, :, j] = 0.5 * v[0] * c
    np.testing.assert_allclose(new[1], expect_S, rtol=1e-14, atol=0)
    np.testing.assert_allclose(out[0], 0.25 * 0.5 * v[0] * c * c, rtol=1e-14)
    assert np.all(np.isnan(new[0]))


def test_null_slots():
    rng = np.random.default_rng(3)
    B = 3
    q, k, v = _single(rng, B)
    pool = rng.standard_normal((3, H, V, K))
    pool[0] = np.nan
    out, new = oracle.gdn_decode(packed(q, k, v), rng.standard_normal((B, H)), rng.standard_normal((B, H)),
                                 rng.standard_normal(H), rng.standard_normal(H), pool,
                                 np.array([0, -4, 2]), H=H, HK=HK, K=K, V=V)
    assert np.all(out[0] == 0) and np.all(out[1] == 0)
    assert np.all(np.isnan(new[0])) and np.array_equal(new[1], pool[1])
    assert not np.array_equal(new[2], pool[2])


def test_rescaled_q_k_leave_the_output():
    rng = np.random.default_rng(4)
    B = 2
    q, k, v = _single(rng, B)
    args = (rng.standard_normal((B, H)), rng.standard_normal((B, H)), rng.standard_normal(H),
            rng.standard_normal(H), rng.standard_normal((3, H, V, K)), np.array([2, 1]))
    o1, p1 = oracle.gdn_decode(packed(q, k, v), *args, H=H, HK=HK, K=K, V=V)
    o2, p2 = oracle.gdn_decode(packed(7.0 * q, 0.5 * k, v), *args, H=H, HK=HK, K=K, V=V)
    # the guard eps = 1e-6 in the norm moves a row of squared norm n by about eps / (2 n)
    np.testing.assert_allclose(o2, o1, rtol=1e-5, atol=2e-6)
    np.testing.assert_allclose(p2, p1, rtol=1e-5, atol=2e-6)
    # an unnormalised variant would differ by the scale factors themselves
    assert np.abs(o2 - o1).max() < 1e-3 * np.abs(o1).max()


def test_steps_match_token_recurrence():
    """T decode steps on slots [2, 5, 1] equal oracle.gdn_forward run on the normalised q, k and the
    transformed gates, started from the same slots."""
    rng = np.random.default_rng(5)
    B, T = 3, 6
    q = rng.standard_normal((B, T, HK, K))
    k = rng.standard_normal((B, T, HK, K))
    v = rng.standard_normal((B, T, H, V))
    rg = rng.standard_normal((B, T, H))
    rb = rng.standard_normal((B, T, H))
    A_log = rng.standard_normal(H) * 0.5
    dt_bias = rng.standard_normal(H) * 0.5
    pool = rng.standard_normal((6, H, V, K)) * 0.3
    idx = np.array([2, 5, 1])
    cur = pool
    outs = []
    for t in range(T):
        o, cur = oracle.gdn_decode(packed(q[:, t], k[:, t], v[:, t]), rg[:, t], rb[:, t], A_log, dt_bias,
                                   cur, idx, H=H, HK=HK, K=K, V=V, scale=0.3)
        outs.append(o)
    outs = np.stack(outs, axis=1)
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + dec.L2_EPS)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + dec.L2_EPS)
    g = -np.exp(A_log) * np.logaddexp(0.0, rg + dt_bias)
    beta = 1.0 / (1.0 + np.exp(-rb))
    ref_o, ref_ht = oracle.gdn_forward(qn, kn, v, g, beta, h0=pool[idx], scale=0.3)
    # oracle.gdn_forward takes float32 inputs: the comparison is at float32 input rounding
    np.testing.assert_allclose(outs, ref_o, rtol=2e-5, atol=2e-6)
    np.testing.assert_allclose(cur[idx], ref_ht, rtol=2e-5, atol=2e-6)
    for s in (0, 3, 4):
        assert np.array_equal(cur[s], pool[s])


def _prepared(rng, B, T):
    """Raw decode inputs for T tokens and the recurrent form's inputs made from them with the decode
    module's helpers (each pinned above)."""
    q = rng.standard_normal((B, T, HK, K))
    k = rng.standard_normal((B, T, HK, K))
    v = rng.standard_normal((B, T, H, V))
    rg = rng.standard_normal((B, T, H))
    rb = rng.standard_normal((B, T, H))
    A_log = rng.standard_normal(H) * 0.5
    dt_bias = rng.standard_normal(H) * 0.5
    qn = np.apply_along_axis(dec.l2_normalise, -1, q)
    kn = np.apply_along_axis(dec.l2_normalise, -1, k)
    g = dec.decay_gate(rg, A_log, dt_bias)
    beta = dec.write_gate(rb)
    return (q, k, v, rg, rb, A_log, dt_bias), (qn, kn, v, g, beta)


def test_paged_recurrent_equals_decode_steps():
    rng = np.random.default_rng(6)
    B, T = 4, 5
    raw, prep = _prepared(rng, B, T)
    pool = rng.standard_normal((7, H, V, K)) * 0.3
    idx = np.array([3, 0, 6, 1])
    fresh = np.array([True, True, False, True])
    out, new = oracle.gdn_recurrent_paged(*prep, pool, idx, fresh, scale=0.3)
    cur, outs = pool, []
    for t in range(T):
        o, cur = oracle.gdn_decode(packed(raw[0][:, t], raw[1][:, t], raw[2][:, t]), raw[3][:, t], raw[4][:, t],
                                   raw[5], raw[6], cur, idx, fresh if t == 0 else None, H=H, HK=HK, K=K, V=V,
                                   scale=0.3)
        outs.append(o)
    outs = np.stack(outs, axis=1)
    np.testing.assert_allclose(out, outs, rtol=2e-5, atol=2e-6)   # gdn_forward reads float32 inputs
    np.testing.assert_allclose(new, cur, rtol=2e-5, atol=2e-6)
    assert np.all(out[1] == 0)                                     # the null sequence
    for s in (0, 2, 4, 5):
        assert np.array_equal(new[s], pool[s])


def test_paged_recurrent_packed_edge_cases():
    """Packed stream: an empty loaded sequence keeps its slot, an empty fresh one zeroes it, a null
    sequence writes nothing and outputs zeros; the others equal separate unpaged runs."""
    rng = np.random.default_rng(7)
    lens = [3, 0, 4, 0, 2]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    _, (qn, kn, v, g, beta) = _prepared(rng, 1, T)
    # float32 values: gdn_forward takes its inputs (h0 included) in float32
    pool = (rng.standard_normal((8, H, V, K)) * 0.3).astype(np.float32).astype(np.float64)
    idx = np.array([5, 2, 0, 7, 1])
    fresh = np.array([True, True, True, False, False])
    out, new = oracle.gdn_recurrent_paged(qn, kn, v, g, beta, pool, idx, fresh, cu_seqlens=cu, scale=0.5)
    assert np.array_equal(new[2], pool[2])                 # empty, loaded: unchanged
    assert np.all(new[7] == 0)                             # empty, fresh: zeroed
    assert np.all(out[0, cu[2]:cu[3]] == 0)                # null sequence
    for s in (0, 3, 4, 6):
        assert np.array_equal(new[s], pool[s])
    for n, (slot, init) in enumerate(zip(idx, fresh)):
        if slot <= 0 or lens[n] == 0:
            continue
        sl = slice(cu[n], cu[n + 1])
        h0 = pool[slot][None] if init else np.zeros((1, H, V, K))
        o1, h1 = oracle.gdn_forward(qn[:, sl], kn[:, sl], v[:, sl], g[:, sl], beta[:, sl], h0=h0, scale=0.5)
        np.testing.assert_allclose(out[:, sl], o1, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(new[slot], h1[0], rtol=1e-12, atol=1e-14)


def test_gate_transform_pins():
    """Closed forms of both kinds: softplus(0) = ln 2 and sigmoid(0) = 1/2; the bounded kind tends
    to lower_bound and to 0 at the two ends; A_log scales the softplus kind's amplitude and the
    bounded kind's slope; per-channel gates with D = 1 equal per-head gates."""
    H = 3
    A = np.log(np.array([1.0, 2.0, 4.0]))
    raw = np.zeros((2, 5, H))
    np.testing.assert_allclose(oracle.gate_transform(raw, A, np.zeros(H), "softplus"),
                               np.broadcast_to(-np.array([1.0, 2.0, 4.0]) * math.log(2.0), raw.shape), rtol=1e-15)
    np.testing.assert_allclose(oracle.gate_transform(raw, A, np.zeros(H), "bounded", lower_bound=-5.0),
                               np.full(raw.shape, -2.5), rtol=1e-15)
    big = np.full((1, 1, H), 60.0)
    np.testing.assert_allclose(oracle.gate_transform(big, A, np.zeros(H), "bounded", lower_bound=-3.0), -3.0, rtol=1e-15)
    assert np.all(np.abs(oracle.gate_transform(-big, A, np.zeros(H), "bounded", lower_bound=-3.0)) < 1e-20)
    # the bias shifts the pre-activation: raw = ln 3, bias = -ln 3 gives the zero point again
    np.testing.assert_allclose(oracle.gate_transform(np.full((1, 1, H), math.log(3.0)), np.zeros(H),
                                                     np.full(H, -math.log(3.0)), "softplus"), -math.log(2.0), rtol=1e-15)
    # the slope of the bounded kind is exp(A_log): sigmoid(2 * ln 3 / 2) = sigmoid(ln 3) = 3/4
    np.testing.assert_allclose(oracle.gate_transform(np.full((1, 1, 1), 0.5 * math.log(3.0)), np.array([math.log(2.0)]),
                                                     np.zeros(1), "bounded", lower_bound=-1.0), -0.75, rtol=1e-15)
    rng = np.random.default_rng(9)
    r = rng.standard_normal((2, 4, H))
    bias = rng.standard_normal(H)
    for kind, lb in (("softplus", None), ("bounded", -5.0)):
        np.testing.assert_array_equal(oracle.gate_transform(r[..., None], A, bias[:, None], kind, lb)[..., 0],
                                      oracle.gate_transform(r, A, bias, kind, lb))


def _kda_inputs(rng, B, T, Hh, Kk, Vv):
    q = rng.standard_normal((B, T, Hh, Kk))
    k = rng.standard_normal((B, T, Hh, Kk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hh, Vv))
    g = -np.logaddexp(0.0, rng.standard_normal((B, T, Hh, Kk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hh))))
    return q, k, v, g, beta


def test_kda_with_uniform_channels_is_the_delta_rule():
    """A per-channel gate equal across channels is the scalar gate: KDA reduces to oracle.gdn_forward."""
    rng = np.random.default_rng(11)
    B, T, Hh, Kk, Vv = 2, 9, 3, 5, 4
    q, k, v, _, beta = _kda_inputs(rng, B, T, Hh, Kk, Vv)
    gs = -np.logaddexp(0.0, rng.standard_normal((B, T, Hh)))
    h0 = rng.standard_normal((B, Hh, Vv, Kk)) * 0.3
    f32 = lambda x: np.asarray(x, np.float32).astype(np.float64)  # gdn_forward reads float32 inputs
    q, k, v, gs, beta, h0 = map(f32, (q, k, v, gs, beta, h0))
    o1, h1 = oracle.kda_forward(q, k, v, np.repeat(gs[..., None], Kk, axis=-1), beta, h0, scale=0.4)
    o2, h2 = oracle.gdn_forward(q, k, v, gs, beta, h0=h0, scale=0.4)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(h1, h2, rtol=1e-12, atol=1e-13)


def test_kda_closed_forms():
    """beta = 0: every key column decays by the product of its own factors and the output reads the
    decayed state; one token from zero: S = beta v k^T and o = scale beta v (k . q)."""
    rng = np.random.default_rng(12)
    B, T, Hh, Kk, Vv = 1, 6, 2, 4, 3
    q, k, v, g, _ = _kda_inputs(rng, B, T, Hh, Kk, Vv)
    h0 = rng.standard_normal((B, Hh, Vv, Kk))
    out, ht = oracle.kda_forward(q, k, v, g, np.zeros((B, T, Hh)), h0, scale=0.5)
    decay = np.exp(np.cumsum(g[0], axis=0))                          # [T, H, K]
    for t in range(T):
        St = h0[0] * decay[t][:, None, :]
        np.testing.assert_allclose(out[0, t], 0.5 * np.einsum("hvk,hk->hv", St, q[0, t]), rtol=1e-12)
    np.testing.assert_allclose(ht[0], h0[0] * decay[-1][:, None, :], rtol=1e-12)
    b1 = np.full((1, 1, Hh), 0.7)
    o1, h1 = oracle.kda_forward(q[:, :1], k[:, :1], v[:, :1], g[:, :1], b1, scale=0.5)
    np.testing.assert_allclose(h1[0], 0.7 * v[0, 0][:, :, None] * k[0, 0][:, None, :], rtol=1e-14)
    np.testing.assert_allclose(o1[0, 0], 0.5 * 0.7 * v[0, 0] * np.sum(k[0, 0] * q[0, 0], -1)[:, None], rtol=1e-13)


def test_kda_packed_equals_separate():
    rng = np.random.default_rng(13)
    lens = [4, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = _kda_inputs(rng, 1, int(cu[-1]), 2, 4, 3)
    h0 = rng.standard_normal((3, 2, 3, 4))
    out, ht = oracle.kda_forward(q, k, v, g, beta, h0, cu_seqlens=cu)
    for n in range(3):
        sl = slice(cu[n], cu[n + 1])
        o1, h1 = oracle.kda_forward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], beta[:, sl], h0[n:n + 1])
        np.testing.assert_array_equal(out[:, sl], o1)
        np.testing.assert_array_equal(ht[n], h1[0])
    np.testing.assert_array_equal(ht[1], h0[1])                     # the empty sequence passes its state


def test_kda_decode_pins():
    """Uniform per-channel raw gates and biases with the softplus kind are GDN's per-head gate: the KDA
    decode equals gdn_decode (H = HK); and T decode steps equal kda_forward on the normalised q, k
    and the transformed gates (each prepared with the decode module's pinned helpers)."""
    rng = np.random.default_rng(14)
    B, Hh, Kk, Vv = 3, 2, 6, 5
    pool = rng.standard_normal((5, Hh, Vv, Kk)) * 0.3
    idx = np.array([4, 0, 2])
    x = rng.standard_normal((B, Hh * (2 * Kk + Vv)))
    rg = rng.standard_normal((B, Hh))
    rb = rng.standard_normal((B, Hh))
    A = rng.standard_normal(Hh) * 0.3
    bias = rng.standard_normal(Hh)
    o1, p1 = oracle.kda_decode(x, np.repeat(rg[..., None], Kk, -1), rb, A, np.repeat(bias[:, None], Kk, -1), pool, idx,
                               H=Hh, K=Kk, V=Vv, kind="softplus", lower_bound=None, scale=0.4)
    o2, p2 = oracle.gdn_decode(x, rg, rb, A, bias, pool, idx, H=Hh, HK=Hh, K=Kk, V=Vv, scale=0.4)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(p1, p2, rtol=1e-13, atol=1e-15)
    # T steps against the KDA token recurrence (bounded kind)
    T = 4
    xs = rng.standard_normal((T, B, Hh * (2 * Kk + Vv)))
    rgs = rng.standard_normal((T, B, Hh, Kk))
    rbs = rng.standard_normal((T, B, Hh))
    dtb = rng.standard_normal((Hh, Kk))
    cur, outs = pool, []
    for t in range(T):
        o, cur = oracle.kda_decode(xs[t], rgs[t], rbs[t], A, dtb, cur, idx, H=Hh, K=Kk, V=Vv, scale=0.4)
        outs.append(o)
    qn = np.apply_along_axis(dec.l2_normalise, -1, xs[..., :Hh * Kk].reshape(T, B, Hh, Kk))
    kn = np.apply_along_axis(dec.l2_normalise, -1, xs[..., Hh * Kk:2 * Hh * Kk].reshape(T, B, Hh, Kk))
    vv = xs[..., 2 * Hh * Kk:].reshape(T, B, Hh, Vv)
    gate = dec.gate_transform(rgs, A, dtb, "bounded", -5.0)
    beta = dec.write_gate(rbs)
    tr = lambda a: np.swapaxes(a, 0, 1)   # [T, B, ...] -> [B, T, ...]
    for b in (0, 2):
        ref_o, ref_h = oracle.kda_forward(tr(qn)[b:b + 1], tr(kn)[b:b + 1], tr(vv)[b:b + 1], tr(gate)[b:b + 1],
                                          tr(beta)[b:b + 1], pool[idx[b]][None], scale=0.4)
        np.testing.assert_allclose(np.stack(outs)[:, b], ref_o[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(cur[idx[b]], ref_h[0], rtol=1e-12, atol=1e-14)
    assert np.all(np.stack(outs)[:, 1] == 0)


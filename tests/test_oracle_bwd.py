"""Pins of the backward oracle (oracle.gdn_backward), all on the CPU.

oracle.gdn_backward differentiates the Gated Delta Rule token loop (attention-gym "Linear Attention", section
"Gated Delta Rule") by reverse-mode, carrying the state cotangent from the last token back to the entry state
(StateFlow Section 2.2, Eq. (6)-(7) carry the gradient of the recurrence backwards in the same way). Every pin
below is independent of that reverse sweep:

* central finite differences of the pinned forward oracle (oracle.gdn_forward) for every element of every
  input, on packed inputs with grouped q/k heads, a ragged tail, an empty sequence, a nonzero initial state
  and a nonzero final-state gradient; the perturbation 2^-12 is exact in float32 at these magnitudes;
* beta = 0: the state only decays, S_t = Gamma_t h0, and every gradient has a closed form written out here;
* do = 0: the loss is <dht, h0 M + S_ext>, so dh0 = dht M^T with M from the pinned summary oracle;
* a sequence cut into segments: the backward of each segment from its true entry state, with the exit-state
  gradient of segment j taken as dh0 of segment j+1, reproduces the unsegmented gradients (the reverse
  counterpart of the exclusive state scan over segment summaries).
"""
import numpy as np
import pytest

import oracle

EPS = 2.0 ** -12


def _inputs(rng, B, T, H, HK, K, V, N=None, h0=True, dht=True):
    n = B if N is None else N
    q = rng.standard_normal((B, T, HK, K)).astype(np.float32)
    k = rng.standard_normal((B, T, HK, K))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, T, H, V)).astype(np.float32)
    g = (-np.log1p(np.exp(rng.standard_normal((B, T, H)) + 0.5))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    d = dict(q=q, k=k, v=v, g=g, beta=beta,
             h0=(0.5 * rng.standard_normal((n, H, V, K))).astype(np.float32) if h0 else None,
             do=rng.standard_normal((B, T, H, V)).astype(np.float32),
             dht=rng.standard_normal((n, H, V, K)).astype(np.float32) if dht else None)
    return d


def _loss(d, cu, scale):
    out, ht = oracle.gdn_forward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], cu_seqlens=cu, scale=scale)
    do = d["do"].astype(np.float64)
    valid = ~np.isnan(out)
    L = float(np.sum(np.where(valid, out, 0.0) * do))
    if d["dht"] is not None:
        L += float(np.sum(ht * d["dht"].astype(np.float64)))
    return L


def test_backward_matches_central_differences():
    rng = np.random.default_rng(7)
    lens = [5, 0, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1]) + 2                       # two tokens past the last sequence
    B, H, HK, K, V = 1, 4, 2, 4, 3
    d = _inputs(rng, B, T, H, HK, K, V, N=len(lens))
    scale = 0.4
    gr = oracle.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["h0"], d["dht"],
                             cu_seqlens=cu, scale=scale)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}
    active = np.zeros(T, dtype=bool)
    active[:cu[-1]] = True
    for x, gx in names.items():
        a = d[x]
        fd = np.zeros(a.shape)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            if x != "h0" and not active[idx[1]]:
                continue
            orig = a[idx]
            a[idx] = orig + np.float32(EPS)
            lp = _loss(d, cu, scale)
            a[idx] = orig - np.float32(EPS)
            lm = _loss(d, cu, scale)
            a[idx] = orig
            fd[idx] = (lp - lm) / (2 * EPS)
        got = gr[gx]
        if x != "h0":
            got = got[:, active]
            fd = fd[:, active]
            assert np.isnan(gr[gx][:, ~active]).all(), f"{gx}: tokens outside every sequence must stay untouched"
        err = np.abs(got - fd).max()
        assert err <= 1e-6 * (1.0 + np.abs(fd).max()), f"{gx}: max |grad - central difference| = {err:.3e}"
    # the empty sequence passes its state through: dh0 = dht
    np.testing.assert_array_equal(gr["dh0"][1], d["dht"][1].astype(np.float64))


def test_backward_beta_zero_closed_form():
    # beta = 0: S_t = Gamma_t h0 with Gamma_t = exp(sum_{i<=t} g_i), o_t = scale Gamma_t h0 q_t. With
    # L = sum_t do_t . o_t + <dht, S_T> and the state gradient dS_t = sum_{tau>=t} scale (Gamma_tau / Gamma_t)
    # do_tau q_tau^T + (Gamma_T / Gamma_t) dht:
    #   dq_t = scale Gamma_t h0^T do_t;  dk = dv = 0;
    #   dg_t = sum_{tau>=t} scale Gamma_tau do_tau . (h0 q_tau) + Gamma_T <dht, h0>;
    #   dbeta_t = (dS_t k_t) . (v_t - Gamma_t h0 k_t);  dh0 = sum_t scale Gamma_t do_t q_t^T + Gamma_T dht.
    rng = np.random.default_rng(11)
    B, T, H, K, V = 1, 13, 2, 5, 4
    d = _inputs(rng, B, T, H, H, K, V)
    d["beta"][:] = 0.0
    scale = 0.7
    gr = oracle.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["h0"], d["dht"], scale=scale)
    f = lambda a: a.astype(np.float64)
    for h in range(H):
        q, k, v, g, do = f(d["q"][0, :, h]), f(d["k"][0, :, h]), f(d["v"][0, :, h]), f(d["g"][0, :, h]), f(d["do"][0, :, h])
        h0, dht = f(d["h0"][0, h]), f(d["dht"][0, h])
        Gam = np.exp(np.cumsum(g))
        dq = scale * Gam[:, None] * (do @ h0)
        dgt = np.array([sum(scale * Gam[tau] * do[tau] @ (h0 @ q[tau]) for tau in range(t, T)) + Gam[-1] * np.sum(dht * h0)
                        for t in range(T)])
        dS = [sum(scale * Gam[tau] / Gam[t] * np.outer(do[tau], q[tau]) for tau in range(t, T)) + Gam[-1] / Gam[t] * dht
              for t in range(T)]
        db = np.array([(dS[t] @ k[t]) @ (v[t] - Gam[t] * h0 @ k[t]) for t in range(T)])
        dh0 = sum(scale * Gam[t] * np.outer(do[t], q[t]) for t in range(T)) + Gam[-1] * dht
        np.testing.assert_allclose(gr["dq"][0, :, h], dq, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(gr["dg"][0, :, h], dgt, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(gr["dbeta"][0, :, h], db, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(gr["dh0"][0, h], dh0, rtol=1e-12, atol=1e-13)
    assert np.abs(gr["dk"]).max() == 0.0 and np.abs(gr["dv"]).max() == 0.0


def test_backward_dh0_through_summary():
    # do = 0: the loss is <dht, h0 M + S_ext> (the range is affine in its entry state), so dh0 = dht M^T
    rng = np.random.default_rng(12)
    lens = [70, 1, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, H, K, V = int(cu[-1]), 2, 6, 5
    d = _inputs(rng, 1, T, H, H, K, V, N=len(lens))
    d["do"][:] = 0.0
    gr = oracle.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["h0"], d["dht"], cu_seqlens=cu)
    M, _ = oracle.gdn_summary(d["k"], d["v"], d["g"], d["beta"], cu_seqlens=cu)
    want = np.einsum("nhvj,nhkj->nhvk", d["dht"].astype(np.float64), M)
    np.testing.assert_allclose(gr["dh0"], want, rtol=1e-11, atol=1e-12)


def test_segmented_backward_equals_unsegmented():
    rng = np.random.default_rng(13)
    B, T, H, HK, K, V = 1, 150, 2, 1, 8, 6
    d = _inputs(rng, B, T, H, HK, K, V)
    scale = 0.3
    full = oracle.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["h0"], d["dht"], scale=scale)
    cuts = [0, 40, 41, 100, 150]
    # true entry states of the segments by the forward oracle (the oracle takes float32 states, so the
    # carried entry states and state gradients are rounded to float32 at each boundary)
    entry = [d["h0"][0].astype(np.float64)]
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = {x: d[x][:, a:b] for x in ("q", "k", "v", "g", "beta")}
        _, ht = oracle.gdn_forward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], entry[-1][None], scale=scale)
        entry.append(ht[0])
    seg = {x: np.full_like(full[x], np.nan) for x in ("dq", "dk", "dv", "dg", "dbeta")}
    dS = d["dht"][0].astype(np.float64)
    for j in range(len(cuts) - 2, -1, -1):
        a, b = cuts[j], cuts[j + 1]
        sl = {x: d[x][:, a:b] for x in ("q", "k", "v", "g", "beta", "do")}
        gj = oracle.gdn_backward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], sl["do"],
                                 entry[j][None].astype(np.float32), dS[None].astype(np.float32), scale=scale)
        for x in seg:
            seg[x][:, a:b] = gj[x]
        dS = gj["dh0"][0]
    # (tolerances: the float32 rounding of the two carried tensors)
    for x in seg:
        np.testing.assert_allclose(seg[x], full[x], rtol=2e-5, atol=2e-6, err_msg=x)
    np.testing.assert_allclose(dS, full["dh0"][0], rtol=2e-5, atol=2e-6)


def test_grouped_heads_sum_over_value_heads():
    # q/k shared by H/HK value heads: dq and dk are the sums of the gradients of separate copies
    rng = np.random.default_rng(14)
    B, T, H, HK, K, V = 2, 20, 4, 2, 4, 3
    d = _inputs(rng, B, T, H, HK, K, V)
    gr = oracle.gdn_backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], d["h0"], d["dht"], scale=0.5)
    qe = np.repeat(d["q"], H // HK, axis=2)
    ke = np.repeat(d["k"], H // HK, axis=2)
    ge = oracle.gdn_backward(qe, ke, d["v"], d["g"], d["beta"], d["do"], d["h0"], d["dht"], scale=0.5)
    for x in ("dq", "dk"):
        want = ge[x].reshape(B, T, HK, H // HK, K).sum(axis=3)
        np.testing.assert_allclose(gr[x], want, rtol=1e-12, atol=1e-13)
    for x in ("dv", "dg", "dbeta", "dh0"):
        np.testing.assert_allclose(gr[x], ge[x], rtol=1e-12, atol=1e-13)

"""GPU parity of the delta-rule chunk backward (sf_gdn_chunk_bwd through the C ABI) against the float64
oracle (oracle.gdn_backward: the token rule of attention-gym "Linear Attention", section "Gated Delta Rule",
differentiated by reverse-mode; pinned in tests/test_oracle_bwd.py).

Tolerances, per gradient tensor over the tokens of the sequences: float32 inputs, max |x - oracle| <= 1e-4
times max(1, max |oracle|) (the float32 bar of the forward, scaled to the gradient's size); bf16 inputs,
rel_rms <= 2e-2 (the bf16 bar of the forward) per tensor and per (sequence, head).
"""
import sys

import numpy as np
import pytest
import torch

import chunked_linear_recurrence_amd as sf
import workloads as wl

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_rms(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def np32(t):
    return None if t is None else t.detach().float().cpu().numpy()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sf.lib()
    return torch.device("cuda:0")


def run_case(dev, oracle, d, do, dht, cu=None, scale=None, heads_check=None):
    """GPU backward and oracle on the same inputs; returns dicts of numpy arrays (active tokens only
    compared by the caller)."""
    c = lambda t: None if t is None else t.to(dev).contiguous()
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).to(dev)
    out = sf.gdn_chunk_bwd(c(d["q"]), c(d["k"]), c(d["v"]), c(d["g"]), c(d["beta"]), c(do), c(d["h0"]), c(dht),
                           cu_seqlens=cu_d, scale=scale)
    torch.cuda.synchronize()
    gpu = dict(zip(NAMES, (np32(x) for x in out)))
    ref = oracle.gdn_backward(np32(d["q"]), np32(d["k"]), np32(d["v"]), np32(d["g"]), np32(d["beta"]), np32(do),
                              np32(d["h0"]), np32(dht), cu_seqlens=cu, scale=scale)
    return gpu, ref


def check(gpu, ref, bf16, label, cu=None, T=None):
    if cu is None:
        act = np.s_[:]
    else:
        act = np.s_[:, :int(cu[-1])]
    for x in NAMES:
        g, r = gpu[x], ref[x]
        if x != "dh0":
            g, r = g[act], r[act]
        assert np.isfinite(g).all(), f"{label} {x}: non-finite values"
        if bf16:
            e = rel_rms(g, r)
            say(f"  {label} {x}: rel_rms {e:.2e}")
            assert e <= 2e-2, f"{label} {x}: rel_rms {e:.3e}"
        else:
            e = float(np.max(np.abs(g - r))) if r.size else 0.0
            bound = 1e-4 * max(1.0, float(np.max(np.abs(r))) if r.size else 1.0)
            say(f"  {label} {x}: max abs {e:.2e} (bound {bound:.2e})")
            assert e <= bound, f"{label} {x}: max abs {e:.3e} > {bound:.3e}"


def test_bwd_tiny_fp32(dev, oracle):
    # the tiny configuration's shape (B=1, T=256, H=2, K=V=64, float32), with an initial state and a
    # final-state gradient
    say("case: backward, B=1 T=256 H=2 K=V=64 float32, h0 and dht")
    d = wl.delta_rule_inputs(B=1, T=256, H=2, K=64, V=64, dtype=torch.float32, seed=201, h0_std=0.1)
    u = wl.upstream_grads(d["rng"], B=1, T=256, H=2, V=64, K=64, N=1, dtype=torch.float32)
    gpu, ref = run_case(dev, oracle, d, u["do"], u["dht"], scale=0.125)
    check(gpu, ref, False, "tiny")


@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 64, 64), (torch.float32, 128, 64), (torch.float32, 64, 128),
                                       (torch.bfloat16, 128, 128), (torch.bfloat16, 64, 64)])
def test_bwd_varlen_packed(dev, oracle, dtype, K, V):
    # packed sequences: an empty one, a single-token one, partial chunks and exact multiples of 64, tokens past
    # the last sequence; no initial state for some (h0 given for all: N x H states)
    lens = [0, 1, 64, 130, 5, 200, 0, 63]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1]) + 9
    H = 3
    say(f"case: backward packed {dtype} K={K} V={V} lengths {lens}")
    d = wl.delta_rule_inputs(B=1, T=T, H=H, K=K, V=V, dtype=dtype, seed=202 + K + V, h0_std=0.1, N=len(lens))
    u = wl.upstream_grads(d["rng"], B=1, T=T, H=H, V=V, K=K, N=len(lens), dtype=dtype)
    gpu, ref = run_case(dev, oracle, d, u["do"], u["dht"], cu=cu)
    check(gpu, ref, dtype == torch.bfloat16, "packed", cu=cu)
    # an empty sequence passes the state gradient through
    np.testing.assert_array_equal(gpu["dh0"][0], np32(u["dht"])[0])


def test_bwd_no_initial_state_no_dht(dev, oracle):
    say("case: backward without h0 and without dht, B=2 T=200 H=2 K=V=128 bf16")
    d = wl.delta_rule_inputs(B=2, T=200, H=2, K=128, V=128, seed=211)
    u = wl.upstream_grads(d["rng"], B=2, T=200, H=2, V=128, K=128, N=2, dht=False)
    gpu, ref = run_case(dev, oracle, d, u["do"], None)
    check(gpu, ref, True, "no-h0")


def test_bwd_dense_full_size(dev, oracle):
    # the dense prefill configuration (B=2, T=4096, H=16, K=V=128, bf16, h0 ~ N(0, 0.02)), every head, with
    # do ~ N(0,1) and dht ~ N(0,1); also per (sequence, head)
    w = wl.dense_gdn()
    say(f"case: backward at the dense prefill size B={w.B} T={w.T} H={w.H} K=V={w.K} bf16")
    d = dict(q=w.q, k=w.k, v=w.v, g=w.g, beta=w.beta, h0=w.h0)
    u = wl.upstream_grads(np.random.default_rng(212), B=w.B, T=w.T, H=w.H, V=w.V, K=w.K, N=w.B)
    gpu, ref = run_case(dev, oracle, d, u["do"], u["dht"], scale=w.scale)
    check(gpu, ref, True, "dense")
    worst = 0.0
    for x in NAMES:
        for n in range(w.B):
            for h in range(w.H):
                g_ = gpu[x][n, h] if x == "dh0" else gpu[x][n, :, h]
                r_ = ref[x][n, h] if x == "dh0" else ref[x][n, :, h]
                e = rel_rms(g_, r_)
                worst = max(worst, e)
                assert e <= 2e-2, f"dense {x} seq {n} head {h}: rel_rms {e:.3e}"
    say(f"  worst per (sequence, head) rel_rms {worst:.2e}")

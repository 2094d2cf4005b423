"""GPU parity of the Kimi Delta Attention chunk forward (sf_kda_chunk_fwd through the C ABI) against the
float64 token-by-token oracle (oracle.kda_forward: attention-gym "Linear Attention", section "Kimi Delta
Attention"; pinned in tests/test_oracle_decode.py).

Tolerances as the delta-rule chunk forward: float32 inputs, max |x - oracle| <= 1e-4 on outputs and final
states; bf16 inputs, rel_rms <= 2e-2 per tensor and per (sequence, head)."""
import sys

import numpy as np
import pytest
import torch

import chunked_linear_recurrence_amd as sf
import workloads as wl

pytestmark = pytest.mark.gpu


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


def run(dev, oracle, d, cu=None, scale=None):
    c = lambda t: None if t is None else t.to(dev).contiguous()
    cu_d = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).to(dev)
    o, ht = sf.kda_chunk_fwd(c(d["q"]), c(d["k"]), c(d["v"]), c(d["g"]), c(d["beta"]), c(d["h0"]), cu_seqlens=cu_d,
                             scale=scale, output_final_state=True)
    torch.cuda.synchronize()
    ro, rh = oracle.kda_forward(np32(d["q"]), np32(d["k"]), np32(d["v"]), np32(d["g"]), np32(d["beta"]), np32(d["h0"]),
                                cu_seqlens=cu, scale=scale)
    return np32(o), np32(ht), ro, rh


def spans(B, T, cu):
    if cu is None:
        return [(n, n, 0, T) for n in range(B)]
    return [(n, 0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]


def check(o, ht, ro, rh, bf16, label, B, T, H, cu=None):
    assert np.isfinite(ht).all()
    for n, b, a, e in spans(B, T, cu):
        assert np.isfinite(o[b, a:e]).all(), f"{label}: non-finite output in sequence {n}"
        for h in range(H):
            units = [("o", o[b, a:e, h], ro[b, a:e, h]), ("ht", ht[n, h], rh[n, h])]
            for name, x, r in units:
                if r.size == 0:
                    continue
                if bf16:
                    err = rel_rms(x, r) if np.linalg.norm(r) > 0 else float(np.abs(x).max())
                    assert err <= 2e-2, f"{label} {name} seq {n} head {h}: rel_rms {err:.3e}"
                else:
                    err = float(np.max(np.abs(x - r)))
                    assert err <= 1e-4, f"{label} {name} seq {n} head {h}: max abs {err:.3e}"
    act = np.concatenate([o[b, a:e].reshape(-1) for _, b, a, e in spans(B, T, cu)])
    ref = np.concatenate([ro[b, a:e].reshape(-1) for _, b, a, e in spans(B, T, cu)])
    say(f"  {label}: output rel_rms {rel_rms(act, ref):.2e}  final state rel_rms {rel_rms(ht, rh):.2e}")


@pytest.mark.parametrize("K,V", [(64, 64), (128, 64), (128, 128)])
def test_kda_chunk_fp32_small(dev, oracle, K, V):
    say(f"case: KDA chunk float32 B=2 T=200 H=2 K={K} V={V}, h0")
    d = wl.kda_inputs(B=2, T=200, H=2, K=K, V=V, dtype=torch.float32, seed=301 + K + V, h0_std=0.1)
    o, ht, ro, rh = run(dev, oracle, d)
    check(o, ht, ro, rh, False, "fp32", 2, 200, 2)


@pytest.mark.parametrize("K,V", [(64, 64), (128, 64), (128, 128)])
def test_kda_chunk_bf16_shapes(dev, oracle, K, V):
    # every (K, V) the bf16 path accepts, packed with partial chunks and an empty sequence
    lens = [200, 0, 37, 64, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    say(f"case: KDA chunk bf16 packed K={K} V={V} H=2 lengths {lens}, h0")
    d = wl.kda_inputs(B=1, T=T, H=2, K=K, V=V, seed=310 + K + V, h0_std=0.1, N=len(lens))
    o, ht, ro, rh = run(dev, oracle, d, cu=cu)
    check(o, ht, ro, rh, True, f"bf16 K={K} V={V}", 1, T, 2, cu=cu)


def test_kda_chunk_strong_decay_fp32(dev, oracle):
    # per-channel gates around -4 per token (decays to e^-256 within a chunk): no overflow, no NaN
    say("case: KDA chunk float32, strong per-channel decay (g = -softplus(N(0,1) + 4))")
    d = wl.kda_inputs(B=1, T=300, H=2, K=128, V=128, dtype=torch.float32, seed=305, gate_shift=4.0, h0_std=0.1)
    o, ht, ro, rh = run(dev, oracle, d)
    check(o, ht, ro, rh, False, "strong-decay", 1, 300, 2)


@pytest.mark.parametrize("shift,label", [(30.0, "every diagonal block pairwise"), (3.6, "mixed")])
def test_kda_chunk_decay_range_paths(dev, oracle, shift, label):
    # The prep forms a diagonal 16-token block through a reference token when the block's per-channel decay
    # range is at most 64 and with the pairwise decays otherwise: g around -30 per token sends every block to
    # the pairwise form; g around -3.6 puts a block's 15-step ranges near 55, past 64 on some channels of
    # some blocks, so both forms run within one launch.
    say(f"case: KDA chunk float32, g = -softplus(N(0,1) + {shift}) ({label})")
    d = wl.kda_inputs(B=1, T=256, H=2, K=128, V=64, dtype=torch.float32, seed=308 + int(shift), gate_shift=shift,
                      h0_std=0.1)
    o, ht, ro, rh = run(dev, oracle, d)
    check(o, ht, ro, rh, False, f"decay-range {shift}", 1, 256, 2)


def test_kda_chunk_packed_bf16(dev, oracle):
    lens = [0, 1, 64, 130, 5, 700, 0, 63]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1]) + 7
    say(f"case: KDA chunk bf16 packed K=V=128 H=4 lengths {lens}, h0")
    d = wl.kda_inputs(B=1, T=T, H=4, K=128, V=128, seed=306, h0_std=0.1, N=len(lens))
    o, ht, ro, rh = run(dev, oracle, d, cu=cu)
    check(o, ht, ro, rh, True, "packed", 1, T, 4, cu=cu)
    # an empty sequence passes its state through
    np.testing.assert_array_equal(ht[0], np32(d["h0"])[0])


@pytest.mark.parametrize("h0", [False, True])
def test_kda_chunk_dense_full_size(dev, oracle, h0):
    # the dense prefill shape (B=2, T=4096, H=16, K=V=128, bf16), every sequence and head
    say(f"case: KDA chunk bf16 dense B=2 T=4096 H=16 K=V=128, h0={h0}")
    d = wl.kda_inputs(B=2, T=4096, H=16, K=128, V=128, seed=307, h0_std=0.02 if h0 else None)
    o, ht, ro, rh = run(dev, oracle, d)
    check(o, ht, ro, rh, True, "dense", 2, 4096, 16)

"""GPU parity of the one-token paged decode (sf_gdn_decode through the C ABI) against the float64
decode oracle (oracle/decode.py, pinned in tests/test_oracle_decode.py).

Tolerances as for the chunk path: float32 rows and pool, max |x - oracle| <= 1e-4 on outputs and
on every advanced slot; bf16 rows (float32 or bf16 pool), rel_rms <= 2e-2 per tensor. Slots no
row names, and the slots of null rows, must come back bit-identical.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import chunked_linear_recurrence_amd as sf
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

FP32_ATOL = 1e-4
BF16_RTOL = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_rms(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sf.lib()
    return torch.device("cuda:0")


def run_gpu(d, dev, scale, steps=1, pool=None):
    """Run `steps` decode calls on the same rows; returns (out of the last call, pool) on the host."""
    g = {n: (None if d[n] is None else d[n].to(dev).contiguous())
         for n in ("packed_qkv", "raw_gate", "raw_beta", "A_log", "dt_bias", "state_indices", "has_initial_state")}
    pool = d["pool"].to(dev).contiguous() if pool is None else pool
    out = None
    for i in range(steps):  # the fresh-slot mask applies to the first call only
        out = sf.gdn_decode(g["packed_qkv"], g["raw_gate"], g["raw_beta"], g["A_log"], g["dt_bias"], pool,
                            g["state_indices"], has_initial_state=g["has_initial_state"] if i == 0 else None,
                            scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()[0], pool


def run_oracle(d, H, HK, K, V, scale, steps=1):
    f = wl.to_f32
    pool = f(d["pool"])
    fresh = None if d["has_initial_state"] is None else d["has_initial_state"].numpy()
    out = None
    for i in range(steps):
        out, pool = oracle.gdn_decode(f(d["packed_qkv"]), f(d["raw_gate"]), f(d["raw_beta"]), f(d["A_log"]),
                                      f(d["dt_bias"]), pool, d["state_indices"].numpy(),
                                      fresh if i == 0 else None, H=H, HK=HK, K=K, V=V, scale=scale)
    return out, pool


def check(out, pool, ref_out, ref_pool, d, fp32, tag):
    idx = d["state_indices"].numpy()
    active = sorted(int(s) for s in idx if s > 0)
    untouched = [s for s in range(pool.shape[0]) if s not in set(active)]
    p0 = wl.to_f32(d["pool"])
    for s in untouched:
        assert np.array_equal(pool[s], p0[s], equal_nan=True), f"{tag}: slot {s} was written"
    null_rows = [b for b in range(len(idx)) if idx[b] <= 0]
    assert np.all(out[null_rows] == 0), f"{tag}: null rows must give zero output"
    got_p, ref_p = pool[active], ref_pool[active]
    if fp32:
        eo, ep = float(np.max(np.abs(out - ref_out))), float(np.max(np.abs(got_p - ref_p)))
        say(f"{tag}: max|o|err {eo:.3g}  max|S|err {ep:.3g}")
        assert eo <= FP32_ATOL and ep <= FP32_ATOL
    else:
        eo, ep = rel_rms(out, ref_out), rel_rms(got_p, ref_p)
        say(f"{tag}: rel_rms o {eo:.3g}  S {ep:.3g}")
        assert eo <= BF16_RTOL and ep <= BF16_RTOL


CASES = [
    # name, dtype, pool dtype, B, H, HK, K, V, nulls, fresh
    ("bf16-f32pool-gqa", torch.bfloat16, torch.float32, 37, 8, 4, 128, 128, 3, 4),
    ("f32-k64", torch.float32, torch.float32, 16, 4, 4, 64, 64, 2, 2),
    ("bf16-bf16pool-v64", torch.bfloat16, torch.bfloat16, 24, 6, 2, 128, 64, 1, 3),
    ("f32-k256-v32", torch.float32, torch.float32, 9, 2, 1, 256, 32, 1, 1),
    ("f32-k64-v128-gqa", torch.float32, torch.float32, 5, 8, 2, 64, 128, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_vs_oracle(dev, case):
    name, dt, pdt, B, H, HK, K, V, nulls, fresh = case
    say(f"decode {name}: B={B} H={H} HK={HK} K={K} V={V}")
    d = wl.decode_inputs(B=B, H=H, HK=HK, K=K, V=V, dtype=dt, pool_dtype=pdt, seed=zlib.crc32(name.encode()) % 1000,
                         num_slots=B + 5, n_null=nulls, n_fresh=fresh, pool_std=0.3)
    scale = 1.0 / np.sqrt(K)
    out, pool = run_gpu(d, dev, scale)
    ref_out, ref_pool = run_oracle(d, H, HK, K, V, scale)
    check(out, pool.float().cpu().numpy(), ref_out, ref_pool, d, dt == torch.float32 and pdt == torch.float32, name)


def test_decode_steps_carry_the_state(dev):
    """Eight calls on the same rows: each advances the same slots from where the last left them."""
    B, H, HK, K, V = 12, 4, 2, 128, 128
    d = wl.decode_inputs(B=B, H=H, HK=HK, K=K, V=V, dtype=torch.float32, seed=7, num_slots=20, n_null=2,
                         n_fresh=3, pool_std=0.3)
    say("decode: eight steps")
    out, pool = run_gpu(d, dev, 0.2, steps=8)
    ref_out, ref_pool = run_oracle(d, H, HK, K, V, 0.2, steps=8)
    check(out, pool.float().cpu().numpy(), ref_out, ref_pool, d, True, "eight steps")


def test_decode_padded_slots(dev):
    """Slots with padding between them (each [H, V, K] block dense): the padding is never touched."""
    B, H, HK, K, V = 6, 2, 2, 64, 64
    d = wl.decode_inputs(B=B, H=H, HK=HK, K=K, V=V, dtype=torch.float32, seed=8, num_slots=8, pool_std=0.3)
    big = torch.full((8, H + 1, V, K), 7.0, dtype=torch.float32, device=dev)
    big[:, :H] = d["pool"].to(dev)
    view = big[:, :H]
    assert view.stride(0) == (H + 1) * V * K
    say("decode: padded slots")
    out, _ = run_gpu(d, dev, 0.125, pool=view)
    ref_out, ref_pool = run_oracle(d, H, HK, K, V, 0.125)
    check(out, view.cpu().numpy(), ref_out, ref_pool, d, True, "padded slots")
    assert torch.all(big[:, H] == 7.0)


def test_decode_full_size(dev):
    """The bench's decode workload (256 rows, H=32, K=V=128, bf16 rows, float32 pool), every row and
    head against the oracle."""
    w = wl.decode_gdn()
    say("decode: full-size workload")
    d = {n: getattr(w, n) for n in ("packed_qkv", "raw_gate", "raw_beta", "A_log", "dt_bias", "pool",
                                    "state_indices", "has_initial_state")}
    out, pool = run_gpu(d, dev, w.scale)
    ref_out, ref_pool = run_oracle(d, w.H, w.HK, w.K, w.V, w.scale)
    check(out, pool.cpu().numpy(), ref_out, ref_pool, d, False, "decode_gdn")

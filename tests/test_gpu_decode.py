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


# ---------------------------------------------------------------------------------------------
# token-by-token forward (sf_gdn_recurrent_fwd)
# ---------------------------------------------------------------------------------------------

REC_CASES = [
    # name, dtype, B, T, H, HK, K, V, h0, lengths (packed) or None
    ("f32-k64-h0", torch.float32, 2, 37, 4, 2, 64, 64, True, None),
    ("bf16-k128-h0", torch.bfloat16, 2, 50, 4, 4, 128, 128, True, None),
    ("f32-k256-v32", torch.float32, 1, 9, 2, 1, 256, 32, False, None),
    ("bf16-packed", torch.bfloat16, 1, 0, 4, 2, 128, 64, True, [5, 0, 17, 1, 30]),
]


@pytest.mark.parametrize("case", REC_CASES, ids=[c[0] for c in REC_CASES])
def test_recurrent_vs_oracle(dev, case):
    name, dt, B, T, H, HK, K, V, with_h0, lens = case
    cu = None
    if lens is not None:
        T = int(sum(lens)) + 3                       # three rows past the terminal offset stay unwritten
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    N = B if lens is None else len(lens)
    say(f"recurrent {name}: B={B} T={T} H={H} HK={HK} K={K} V={V} N={N}")
    d = wl.delta_rule_inputs(B=B, T=T, H=H, HK=HK, K=K, V=V, dtype=dt, seed=zlib.crc32(name.encode()) % 1000,
                             gate_shift=1.0, h0_std=0.3 if with_h0 else None, N=N)
    g = {n: (None if d[n] is None else d[n].to(dev).contiguous()) for n in ("q", "k", "v", "g", "beta", "h0")}
    o, ht = sf.gdn_recurrent_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"],
                                 cu_seqlens=None if cu is None else cu.to(dev), scale=0.3, output_final_state=True)
    torch.cuda.synchronize()
    f = wl.to_f32
    ref_o, ref_ht = oracle.gdn_forward(f(d["q"]), f(d["k"]), f(d["v"]), f(d["g"]), f(d["beta"]), f(d["h0"]),
                                       cu_seqlens=None if cu is None else cu.numpy(), scale=0.3)
    o = o.float().cpu().numpy()
    ht = ht.cpu().numpy()
    if cu is not None:
        end = int(cu[-1])
        o, ref_o = o[:, :end], ref_o[:, :end]
    if dt == torch.float32:
        eo, eh = float(np.max(np.abs(o - ref_o))), float(np.max(np.abs(ht - ref_ht)))
        say(f"{name}: max|o|err {eo:.3g}  max|ht|err {eh:.3g}")
        assert eo <= FP32_ATOL and eh <= FP32_ATOL
    else:
        eo, eh = rel_rms(o, ref_o), rel_rms(ht, ref_ht)
        say(f"{name}: rel_rms o {eo:.3g}  ht {eh:.3g}")
        assert eo <= BF16_RTOL and eh <= BF16_RTOL


PAGED_CASES = [
    # name, dtype, pool dtype, B, T, lengths or None, nulls, fresh
    ("f32-dense", torch.float32, torch.float32, 6, 12, None, 1, 2),
    ("bf16-bf16pool", torch.bfloat16, torch.bfloat16, 5, 20, None, 1, 1),
    ("bf16-packed-empty", torch.bfloat16, torch.float32, 1, 0, [7, 0, 0, 13, 4, 0], 1, 2),
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[c[0] for c in PAGED_CASES])
def test_recurrent_paged_vs_oracle(dev, case):
    name, dt, pdt, B, T, lens, nulls, fresh_n = case
    H, HK, K, V = 4, 2, 128, 128
    cu = None
    if lens is not None:
        T = int(sum(lens))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    N = B if lens is None else len(lens)
    say(f"recurrent paged {name}: N={N} T={T}")
    seed = zlib.crc32(name.encode()) % 1000
    d = wl.delta_rule_inputs(B=B, T=T, H=H, HK=HK, K=K, V=V, dtype=dt, seed=seed, gate_shift=1.0)
    p = wl.decode_inputs(B=N, H=H, HK=HK, K=K, V=V, dtype=dt, pool_dtype=pdt, seed=seed + 1, num_slots=N + 4,
                         n_null=nulls, n_fresh=fresh_n, pool_std=0.3)
    pool = p["pool"].to(dev).contiguous()
    g = {n: d[n].to(dev).contiguous() for n in ("q", "k", "v", "g", "beta")}
    fresh = p["has_initial_state"]
    o, none = sf.gdn_recurrent_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], pool,
                                   cu_seqlens=None if cu is None else cu.to(dev), scale=0.25,
                                   state_indices=p["state_indices"].to(dev),
                                   has_initial_state=None if fresh is None else fresh.to(dev))
    assert none is None
    torch.cuda.synchronize()
    f = wl.to_f32
    ref_o, ref_pool = oracle.gdn_recurrent_paged(f(d["q"]), f(d["k"]), f(d["v"]), f(d["g"]), f(d["beta"]),
                                                 f(p["pool"]), p["state_indices"].numpy(),
                                                 None if fresh is None else fresh.numpy(),
                                                 cu_seqlens=None if cu is None else cu.numpy(), scale=0.25)
    o = o.float().cpu().numpy()
    got_pool = pool.float().cpu().numpy()
    idx = p["state_indices"].numpy()
    active = sorted(int(s) for s in idx if s > 0)
    p0 = f(p["pool"])
    for s in range(got_pool.shape[0]):
        if s not in active:
            assert np.array_equal(got_pool[s], p0[s]), f"slot {s} was written"
    if dt == torch.float32 and pdt == torch.float32:
        eo, ep = float(np.max(np.abs(o - ref_o))), float(np.max(np.abs(got_pool[active] - ref_pool[active])))
        say(f"{name}: max|o|err {eo:.3g}  max|S|err {ep:.3g}")
        assert eo <= FP32_ATOL and ep <= FP32_ATOL
    else:
        eo, ep = rel_rms(o, ref_o), rel_rms(got_pool[active], ref_pool[active])
        say(f"{name}: rel_rms o {eo:.3g}  S {ep:.3g}")
        assert eo <= BF16_RTOL and ep <= BF16_RTOL


def test_recurrent_full_size(dev):
    """The bench's recurrent workload (64 sequences of 16 tokens, H=32, K=V=128, bf16, float32 pool),
    every sequence and head against the oracle."""
    w = wl.recurrent_gdn()
    say("recurrent: full-size workload")
    pool = w.meta["pool"].to(dev).contiguous()
    o, _ = sf.gdn_recurrent_fwd(w.q.to(dev), w.k.to(dev), w.v.to(dev), w.g.to(dev), w.beta.to(dev), pool,
                                state_indices=w.meta["state_indices"].to(dev), scale=w.scale)
    torch.cuda.synchronize()
    f = wl.to_f32
    ref_o, ref_pool = oracle.gdn_recurrent_paged(f(w.q), f(w.k), f(w.v), f(w.g), f(w.beta), f(w.meta["pool"]),
                                                 w.meta["state_indices"].numpy(), scale=w.scale)
    eo = rel_rms(o.float().cpu().numpy(), ref_o)
    ep = rel_rms(pool.cpu().numpy()[1:], ref_pool[1:])
    say(f"recurrent_gdn: rel_rms o {eo:.3g}  S {ep:.3g}")
    assert eo <= BF16_RTOL and ep <= BF16_RTOL
    assert np.array_equal(pool[0].cpu().numpy(), f(w.meta["pool"])[0])


# ---------------------------------------------------------------------------------------------
# chunk forward on a paged state cache (sf_paged_gdn_chunk_fwd)
# ---------------------------------------------------------------------------------------------

PAGED_CHUNK_CASES = [
    # name, dtype, pool dtype, K, B, T, lengths or None, nulls, fresh
    ("bf16-dense", torch.bfloat16, torch.float32, 128, 3, 150, None, 1, 1),
    ("f32-k64-dense", torch.float32, torch.float32, 64, 2, 70, None, 0, 1),
    ("bf16-packed-bf16pool", torch.bfloat16, torch.bfloat16, 128, 1, 0, [70, 0, 129, 5, 0, 64], 1, 2),
]


@pytest.mark.parametrize("case", PAGED_CHUNK_CASES, ids=[c[0] for c in PAGED_CHUNK_CASES])
def test_paged_chunk_vs_oracle(dev, case):
    name, dt, pdt, K, B, T, lens, nulls, fresh_n = case
    H, HK, V = 4, 2, K
    cu = None
    if lens is not None:
        T = int(sum(lens))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    N = B if lens is None else len(lens)
    say(f"paged chunk {name}: N={N} T={T}")
    seed = zlib.crc32(name.encode()) % 1000
    d = wl.delta_rule_inputs(B=B, T=T, H=H, HK=HK, K=K, V=V, dtype=dt, seed=seed, gate_shift=1.0)
    p = wl.decode_inputs(B=N, H=H, HK=HK, K=K, V=V, dtype=dt, pool_dtype=pdt, seed=seed + 1, num_slots=N + 3,
                         n_null=nulls, n_fresh=fresh_n, pool_std=0.3)
    pool = p["pool"].to(dev).contiguous()
    g = {n: d[n].to(dev).contiguous() for n in ("q", "k", "v", "g", "beta")}
    fresh = p["has_initial_state"]
    o = sf.paged_gdn_chunk_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], pool, p["state_indices"].to(dev),
                               cu_seqlens=None if cu is None else cu.to(dev),
                               has_initial_state=None if fresh is None else fresh.to(dev), scale=0.25)
    torch.cuda.synchronize()
    f = wl.to_f32
    ref_o, ref_pool = oracle.gdn_recurrent_paged(f(d["q"]), f(d["k"]), f(d["v"]), f(d["g"]), f(d["beta"]),
                                                 f(p["pool"]), p["state_indices"].numpy(),
                                                 None if fresh is None else fresh.numpy(),
                                                 cu_seqlens=None if cu is None else cu.numpy(), scale=0.25)
    o = o.float().cpu().numpy()
    got_pool = pool.float().cpu().numpy()
    idx = p["state_indices"].numpy()
    active = sorted(int(s) for s in idx if s > 0)
    p0 = f(p["pool"])
    for s in range(got_pool.shape[0]):
        if s not in active:
            assert np.array_equal(got_pool[s], p0[s]), f"slot {s} was written"
    for n in range(N):
        if idx[n] <= 0:
            rows = o[n] if cu is None else o[0, cu[n]:cu[n + 1]]
            assert np.all(rows == 0), f"null sequence {n} has nonzero output"
    if dt == torch.float32:
        eo, ep = float(np.max(np.abs(o - ref_o))), float(np.max(np.abs(got_pool[active] - ref_pool[active])))
        say(f"{name}: max|o|err {eo:.3g}  max|S|err {ep:.3g}")
        assert eo <= FP32_ATOL and ep <= FP32_ATOL
    else:
        eo, ep = rel_rms(o, ref_o), rel_rms(got_pool[active], ref_pool[active])
        say(f"{name}: rel_rms o {eo:.3g}  S {ep:.3g}")
        assert eo <= BF16_RTOL and ep <= BF16_RTOL


# ---------------------------------------------------------------------------------------------
# chunk forward with the gate transform fused into Pre (sf_gdn_chunk_fwd_raw_gate)
# ---------------------------------------------------------------------------------------------

RAW_GATE_CASES = [
    # name, dtype, K, B, T, lengths or None, kind, lower bound
    ("bf16-dense-softplus", torch.bfloat16, 128, 2, 300, None, "softplus", None),
    ("bf16-packed-bounded", torch.bfloat16, 64, 1, 0, [100, 0, 37, 200], "bounded", -5.0),
    ("f32-softplus", torch.float32, 64, 1, 130, None, "softplus", None),
]


@pytest.mark.parametrize("case", RAW_GATE_CASES, ids=[c[0] for c in RAW_GATE_CASES])
def test_raw_gate_chunk_vs_oracle(dev, case):
    """The fused path against oracle.gate_transform followed by the token recurrence."""
    name, dt, K, B, T, lens, kind, lb = case
    H, HK, V = 4, 2, K
    cu = None
    if lens is not None:
        T = int(sum(lens))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    N = B if lens is None else len(lens)
    say(f"raw-gate chunk {name}: N={N} T={T}")
    seed = zlib.crc32(name.encode()) % 1000
    d = wl.delta_rule_inputs(B=B, T=T, H=H, HK=HK, K=K, V=V, dtype=dt, seed=seed, h0_std=0.1, N=N)
    gi = wl.gate_inputs(shape=(B, T, H), H=H, dtype=dt, seed=seed + 1)
    g = {n: d[n].to(dev).contiguous() for n in ("q", "k", "v", "beta", "h0")}
    o, ht = sf.gdn_chunk_fwd_raw_gate(g["q"], g["k"], g["v"], gi["raw"].to(dev), gi["A_log"].to(dev),
                                      gi["dt_bias"].to(dev), g["beta"], g["h0"], kind=kind, lower_bound=lb,
                                      cu_seqlens=None if cu is None else cu.to(dev), scale=0.2,
                                      output_final_state=True)
    torch.cuda.synchronize()
    f = wl.to_f32
    gate = oracle.gate_transform(f(gi["raw"]), f(gi["A_log"]), f(gi["dt_bias"]), kind, lb)
    ref_o, ref_ht = oracle.gdn_forward(f(d["q"]), f(d["k"]), f(d["v"]), gate, f(d["beta"]), f(d["h0"]),
                                       cu_seqlens=None if cu is None else cu.numpy(), scale=0.2)
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    if dt == torch.float32:
        eo, eh = float(np.max(np.abs(o - ref_o))), float(np.max(np.abs(ht - ref_ht)))
        say(f"{name}: max|o|err {eo:.3g}  max|ht|err {eh:.3g}")
        assert eo <= FP32_ATOL and eh <= FP32_ATOL
    else:
        eo, eh = rel_rms(o, ref_o), rel_rms(ht, ref_ht)
        say(f"{name}: rel_rms o {eo:.3g}  ht {eh:.3g}")
        assert eo <= BF16_RTOL and eh <= BF16_RTOL


def test_paged_chunk_full_size(dev):
    """The paged_gdn workload (the packed 32768-token stream, H = 32, a float32 pool) at full size: the
    launch has more 16-row slices than two per CU and more Pre units than the GPU holds at once, so it runs
    the per-head chain and the one-wavefront Pre, as bench.py's paged_gdn line does. Every sequence and
    head of the output and every advanced slot against the oracle."""
    w = wl.paged_gdn()
    say(f"paged chunk full size: lengths {w.meta['lengths']}")
    pool = w.meta["pool"].to(dev).contiguous()
    idx = w.meta["state_indices"]
    x = {n: getattr(w, n).to(dev).contiguous() for n in ("q", "k", "v", "g", "beta", "cu_seqlens")}
    o = sf.paged_gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, idx.to(dev),
                               cu_seqlens=x["cu_seqlens"], scale=w.scale)
    torch.cuda.synchronize()
    f = wl.to_f32
    ref_o, ref_pool = oracle.gdn_recurrent_paged(f(w.q), f(w.k), f(w.v), f(w.g), f(w.beta), f(w.meta["pool"]),
                                                 idx.numpy(), cu_seqlens=w.cu_seqlens.numpy(), scale=w.scale)
    o = o.float().cpu().numpy()
    got = pool.cpu().numpy()
    cu = w.cu_seqlens.numpy()
    worst = 0.0
    for n in range(w.N):
        for h in range(w.H):
            e = rel_rms(got[idx[n], h], ref_pool[idx[n], h])
            worst = max(worst, e)
            assert e <= BF16_RTOL, ("slot", n, h, e)
            if cu[n + 1] > cu[n]:
                e = rel_rms(o[0, cu[n]:cu[n + 1], h], ref_o[0, cu[n]:cu[n + 1], h])
                worst = max(worst, e)
                assert e <= BF16_RTOL, ("out", n, h, e)
    assert np.array_equal(got[0], f(w.meta["pool"])[0])  # the null slot is untouched
    say(f"paged chunk full size: worst rel_rms over (sequence, head) {worst:.3g}")


def test_raw_gate_chunk_full_size(dev):
    """sf_gdn_chunk_fwd_raw_gate on the packed 32768-token stream with 32 heads (per-head chain,
    one-wavefront Pre with the gate transform in its gate load), softplus kind, against the oracle's
    gate transform followed by the token recurrence, per (sequence, head)."""
    w = wl.varlen_gdn()
    gi = wl.gate_inputs(shape=(1, w.T, w.H), H=w.H, dtype=torch.bfloat16, seed=123)
    say(f"raw-gate chunk full size: lengths {w.meta['lengths']}")
    x = {n: getattr(w, n).to(dev).contiguous() for n in ("q", "k", "v", "beta", "cu_seqlens")}
    o, ht = sf.gdn_chunk_fwd_raw_gate(x["q"], x["k"], x["v"], gi["raw"].to(dev), gi["A_log"].to(dev),
                                      gi["dt_bias"].to(dev), x["beta"], None, kind="softplus",
                                      cu_seqlens=x["cu_seqlens"], scale=w.scale, output_final_state=True)
    torch.cuda.synchronize()
    f = wl.to_f32
    gate = oracle.gate_transform(f(gi["raw"]), f(gi["A_log"]), f(gi["dt_bias"]), "softplus", None)
    ref_o, ref_ht = oracle.gdn_forward(f(w.q), f(w.k), f(w.v), gate, f(w.beta), cu_seqlens=w.cu_seqlens.numpy(),
                                       scale=w.scale)
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    cu = w.cu_seqlens.numpy()
    worst = 0.0
    for n in range(w.N):
        if cu[n + 1] == cu[n]:
            assert np.all(ht[n] == 0)
            continue
        for h in range(w.H):
            for x_, r_ in ((o[0, cu[n]:cu[n + 1], h], ref_o[0, cu[n]:cu[n + 1], h]), (ht[n, h], ref_ht[n, h])):
                e = rel_rms(x_, r_)
                worst = max(worst, e)
                assert e <= BF16_RTOL, (n, h, e)
    say(f"raw-gate chunk full size: worst rel_rms over (sequence, head) {worst:.3g}")


# ---------------------------------------------------------------------------------------------
# Kimi Delta Attention token by token (sf_kda_recurrent_fwd)
# ---------------------------------------------------------------------------------------------

KDA_CASES = [
    # name, dtype, B, T, H, K, V, h0, lengths (packed) or None
    ("f32-k64-h0", torch.float32, 2, 37, 3, 64, 64, True, None),
    ("bf16-k128-h0", torch.bfloat16, 2, 50, 4, 128, 128, True, None),
    ("bf16-packed", torch.bfloat16, 1, 0, 2, 128, 64, True, [9, 0, 33, 17]),
]


@pytest.mark.parametrize("case", KDA_CASES, ids=[c[0] for c in KDA_CASES])
def test_kda_recurrent_vs_oracle(dev, case):
    name, dt, B, T, H, K, V, with_h0, lens = case
    cu = None
    if lens is not None:
        T = int(sum(lens))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    N = B if lens is None else len(lens)
    say(f"kda {name}: B={B} T={T} H={H} K={K} V={V} N={N}")
    d = wl.kda_inputs(B=B, T=T, H=H, K=K, V=V, dtype=dt, seed=zlib.crc32(name.encode()) % 1000, gate_shift=0.5,
                      h0_std=0.3 if with_h0 else None, N=N)
    g = {n: (None if d[n] is None else d[n].to(dev).contiguous()) for n in ("q", "k", "v", "g", "beta", "h0")}
    o, ht = sf.kda_recurrent_fwd(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"],
                                 cu_seqlens=None if cu is None else cu.to(dev), scale=0.3, output_final_state=True)
    torch.cuda.synchronize()
    f = wl.to_f32
    ref_o, ref_ht = oracle.kda_forward(f(d["q"]), f(d["k"]), f(d["v"]), f(d["g"]), f(d["beta"]), f(d["h0"]),
                                       cu_seqlens=None if cu is None else cu.numpy(), scale=0.3)
    o, ht = o.float().cpu().numpy(), ht.cpu().numpy()
    if dt == torch.float32:
        eo, eh = float(np.max(np.abs(o - ref_o))), float(np.max(np.abs(ht - ref_ht)))
        say(f"{name}: max|o|err {eo:.3g}  max|ht|err {eh:.3g}")
        assert eo <= FP32_ATOL and eh <= FP32_ATOL
    else:
        eo, eh = rel_rms(o, ref_o), rel_rms(ht, ref_ht)
        say(f"{name}: rel_rms o {eo:.3g}  ht {eh:.3g}")
        assert eo <= BF16_RTOL and eh <= BF16_RTOL


def test_kda_recurrent_paged_full_size(dev):
    """The bench's KDA workload (64 sequences of 16 tokens, H=32, K=V=128, bf16, float32 pool), every
    sequence and head against the oracle started from the same slots."""
    w = wl.recurrent_kda()
    say("kda: full-size workload")
    pool = w.meta["pool"].to(dev).contiguous()
    idx = w.meta["state_indices"]
    o, _ = sf.kda_recurrent_fwd(w.q.to(dev), w.k.to(dev), w.v.to(dev), w.g.to(dev), w.beta.to(dev), pool,
                                state_indices=idx.to(dev), scale=w.scale)
    torch.cuda.synchronize()
    f = wl.to_f32
    p0 = f(w.meta["pool"])
    ref_o, ref_ht = oracle.kda_forward(f(w.q), f(w.k), f(w.v), f(w.g), f(w.beta), p0[idx.numpy()], scale=w.scale)
    eo = rel_rms(o.float().cpu().numpy(), ref_o)
    eh = rel_rms(pool.cpu().numpy()[idx.numpy()], ref_ht)
    say(f"recurrent_kda: rel_rms o {eo:.3g}  S {eh:.3g}")
    assert eo <= BF16_RTOL and eh <= BF16_RTOL
    assert np.array_equal(pool[0].cpu().numpy(), p0[0])


# ---------------------------------------------------------------------------------------------
# one-token paged KDA decode (sf_kda_decode)
# ---------------------------------------------------------------------------------------------

KDA_DEC_CASES = [
    # name, dtype, pool dtype, B, H, K, V, nulls, fresh, kind, lower bound
    ("bf16-bounded", torch.bfloat16, torch.float32, 21, 4, 128, 128, 2, 3, "bounded", -5.0),
    ("f32-softplus-k64", torch.float32, torch.float32, 9, 3, 64, 64, 1, 1, "softplus", None),
    ("bf16-bf16pool-k256", torch.bfloat16, torch.bfloat16, 6, 2, 256, 32, 1, 1, "bounded", -3.0),
]


@pytest.mark.parametrize("case", KDA_DEC_CASES, ids=[c[0] for c in KDA_DEC_CASES])
def test_kda_decode_vs_oracle(dev, case):
    name, dt, pdt, B, H, K, V, nulls, fresh, kind, lb = case
    say(f"kda decode {name}: B={B} H={H} K={K} V={V}")
    d = wl.kda_decode_inputs(B=B, H=H, K=K, V=V, dtype=dt, pool_dtype=pdt, seed=zlib.crc32(name.encode()) % 1000,
                             num_slots=B + 4, n_null=nulls, n_fresh=fresh, pool_std=0.3)
    g = {n: (None if d[n] is None else d[n].to(dev).contiguous()) for n in d}
    out = sf.kda_decode(g["packed_qkv"], g["raw_gate"], g["raw_beta"], g["A_log"], g["dt_bias"], g["pool"],
                        g["state_indices"], has_initial_state=g["has_initial_state"], gate_transform=kind,
                        lower_bound=lb, scale=0.2)
    torch.cuda.synchronize()
    f = wl.to_f32
    fr = d["has_initial_state"]
    ref_out, ref_pool = oracle.kda_decode(f(d["packed_qkv"]), f(d["raw_gate"]), f(d["raw_beta"]), f(d["A_log"]),
                                          f(d["dt_bias"]), f(d["pool"]), d["state_indices"].numpy(),
                                          None if fr is None else fr.numpy(), H=H, K=K, V=V, kind=kind,
                                          lower_bound=lb, scale=0.2)
    check(out.float().cpu().numpy()[0], g["pool"].float().cpu().numpy(), ref_out, ref_pool, d,
          dt == torch.float32 and pdt == torch.float32, name)


def test_kda_decode_full_size(dev):
    w = wl.decode_kda()
    say("kda decode: full-size workload")
    d = {n: getattr(w, n) for n in ("packed_qkv", "raw_gate", "raw_beta", "A_log", "dt_bias", "pool",
                                    "state_indices", "has_initial_state")}
    g = {n: (None if d[n] is None else d[n].to(dev).contiguous()) for n in d}
    out = sf.kda_decode(g["packed_qkv"], g["raw_gate"], g["raw_beta"], g["A_log"], g["dt_bias"], g["pool"],
                        g["state_indices"], gate_transform=w.gate_kind, lower_bound=w.lower_bound, scale=w.scale)
    torch.cuda.synchronize()
    f = wl.to_f32
    ref_out, ref_pool = oracle.kda_decode(f(w.packed_qkv), f(w.raw_gate), f(w.raw_beta), f(w.A_log), f(w.dt_bias),
                                          f(w.pool), w.state_indices.numpy(), None, H=w.H, K=w.K, V=w.V,
                                          kind=w.gate_kind, lower_bound=w.lower_bound, scale=w.scale)
    check(out.float().cpu().numpy()[0], g["pool"].cpu().numpy(), ref_out, ref_pool, d, False, "decode_kda")


# ---------------------------------------------------------------------------------------------
# degenerate cases of the token-by-token and paged entry points
# ---------------------------------------------------------------------------------------------

def test_degenerate_token_paths(dev):
    """No rows, no tokens, every row null: the entry points return without touching anything they
    should not, and the states pass through where the pages say so."""
    say("degenerate: empty decode batch, zero-length sequences, all-null paged call")
    H, K, V = 2, 64, 64
    # a decode call with no rows
    d = wl.decode_inputs(B=1, H=H, HK=H, K=K, V=V, dtype=torch.bfloat16, seed=3)
    pool = d["pool"].to(dev)
    before = pool.clone()
    empty = torch.empty((0, 2 * H * K + H * V), dtype=torch.bfloat16, device=dev)
    out = sf.gdn_decode(empty, torch.empty((1, 0, H), dtype=torch.bfloat16, device=dev),
                        torch.empty((1, 0, H), dtype=torch.bfloat16, device=dev), d["A_log"].to(dev),
                        d["dt_bias"].to(dev), pool, torch.empty(0, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert out.shape == (1, 0, H, V) and torch.equal(pool, before)
    # zero-length sequences: the final state is the initial state, bit for bit
    x = wl.delta_rule_inputs(B=2, T=0, H=H, K=K, V=V, dtype=torch.bfloat16, seed=4, h0_std=0.5)
    h0 = x["h0"].to(dev)
    o, ht = sf.gdn_recurrent_fwd(*(x[n].to(dev) for n in ("q", "k", "v", "g", "beta")), h0, output_final_state=True)
    torch.cuda.synchronize()
    assert o.shape[1] == 0 and torch.equal(ht, h0)
    xk = wl.kda_inputs(B=2, T=0, H=H, K=K, V=V, seed=5, h0_std=0.5)
    o, ht = sf.kda_recurrent_fwd(*(xk[n].to(dev) for n in ("q", "k", "v", "g", "beta")), xk["h0"].to(dev),
                                 output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(ht, xk["h0"].to(dev))
    # a paged chunk call whose rows are all null: zero outputs, the pool untouched
    y = wl.delta_rule_inputs(B=3, T=70, H=H, K=K, V=V, dtype=torch.bfloat16, seed=6)
    pool2 = torch.randn(5, H, V, K, device=dev)
    before2 = pool2.clone()
    o = sf.paged_gdn_chunk_fwd(*(y[n].to(dev) for n in ("q", "k", "v", "g", "beta")), pool2,
                               torch.tensor([0, -1, 0], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.equal(pool2, before2)
    # a gate transform of nothing
    g = sf.gate_transform(torch.empty((0, H), dtype=torch.bfloat16, device=dev), d["A_log"].to(dev),
                          d["dt_bias"].to(dev), kind="softplus")
    assert g.shape == (0, H) and g.dtype == torch.float32

"""GPU parity of the HIP path (through the C ABI) against the float64 oracle.

Tolerances (from the statement of the problem): float32 inputs, max |x - oracle|
<= 1e-4 on outputs and final states; bf16 inputs with float32 state,
rel_rms(x, oracle) = ||x - oracle||_2 / ||oracle||_2 <= 2e-2 per tensor over the
active rows. Integer work (chunk table, segment indexing) and the packing
invariants are bit-exact.

Full-size configurations run the GPU exactly as bench.py does and compare every
sequence of a sample of heads against the oracle (each (sequence, head) chain is
independent, so the sample is exact for those heads).
"""
import sys

import numpy as np
import pytest
import torch

import chunked_linear_recurrence_amd as sf
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


def maxabs(x, ref):
    return float(np.max(np.abs(np.asarray(x, np.float64) - ref))) if np.size(ref) else 0.0


def f32(t):
    return None if t is None else t.detach().float().cpu().numpy()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sf.lib()
    return torch.device("cuda:0")


def cuda(t, dev):
    return None if t is None else t.to(dev).contiguous()


def heads_subset(w, heads):
    """Slice a workload's tensors to the given value heads (q/k follow their groups)."""
    grp = w.H // w.HK
    groups = sorted({h // grp for h in heads})
    assert all(h // grp in groups for h in heads)
    # keep whole groups so the grouping stays H/HK
    hs = [g * grp + i for g in groups for i in range(grp)]
    sub = lambda x, idx: None if x is None else x[:, :, idx]
    return dict(q=f32(sub(w.q, groups)), k=f32(sub(w.k, groups)), v=f32(sub(w.v, hs)), g=f32(sub(w.g, hs)),
                beta=f32(sub(w.beta, hs)), h0=None if w.h0 is None else f32(w.h0[:, hs]), hs=hs)


def check_units(name, units):
    """Per-chain gate: units is a list of (label, x, ref); every unit's rel_rms must pass, so a wrong
    head, short sequence or tail is not diluted by the rest of a large tensor."""
    worst = ("", 0.0)
    for label, x, ref in units:
        if np.linalg.norm(ref) == 0:
            assert np.array_equal(np.asarray(x, np.float64), ref), label
            continue
        e = rel_rms(x, ref)
        if e > worst[1]:
            worst = (label, e)
        assert e <= BF16_RTOL, (name, label, e)
    say(f"  {name}: {len(units)} units, worst rel_rms {worst[1]:.3e} ({worst[0]})")


def check_bf16(name, o, ro, ht, rh):
    eo, eh = rel_rms(o, ro), rel_rms(ht, rh)
    say(f"  {name}: rel_rms(o)={eo:.3e} rel_rms(ht)={eh:.3e}")
    assert eo <= BF16_RTOL and eh <= BF16_RTOL, (name, eo, eh)


# ---------------------------------------------------------------------------
# Gated Delta Rule
# ---------------------------------------------------------------------------

def test_tiny_gdn_fp32(dev, oracle):
    say("case: tiny GDN fp32 B=1 T=256 H=2 K=V=64")
    w = wl.tiny_gdn()
    o, ht = sf.gdn_chunk_fwd(cuda(w.q, dev), cuda(w.k, dev), cuda(w.v, dev), cuda(w.g, dev), cuda(w.beta, dev),
                             scale=w.scale, output_final_state=True)
    ro, rh = oracle.gdn_forward(f32(w.q), f32(w.k), f32(w.v), f32(w.g), f32(w.beta), scale=w.scale)
    eo, eh = maxabs(f32(o), ro), maxabs(f32(ht), rh)
    say(f"  max|o-ref|={eo:.3e} max|ht-ref|={eh:.3e}")
    assert eo <= FP32_ATOL and eh <= FP32_ATOL


@pytest.mark.parametrize("T,D,HK,B", [(1, 64, 2, 2), (63, 64, 1, 2), (64, 128, 2, 1), (65, 64, 2, 2),
                                      (200, 128, 1, 2), (333, 64, 2, 1)])
def test_gdn_fp32_sweep(dev, oracle, T, D, HK, B):
    say(f"case: GDN fp32 T={T} K=V={D} H=2 HK={HK} B={B} with h0")
    d = wl.delta_rule_inputs(B=B, T=T, H=2, HK=HK, K=D, V=D, dtype=torch.float32, seed=T + D, h0_std=0.5)
    o, ht = sf.gdn_chunk_fwd(cuda(d["q"], dev), cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev),
                             cuda(d["beta"], dev), cuda(d["h0"], dev), scale=0.3, output_final_state=True)
    ro, rh = oracle.gdn_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(d["beta"]), f32(d["h0"]),
                                scale=0.3)
    eo, eh = maxabs(f32(o), ro), maxabs(f32(ht), rh)
    say(f"  max|o-ref|={eo:.3e} max|ht-ref|={eh:.3e}")
    assert eo <= FP32_ATOL and eh <= FP32_ATOL


@pytest.mark.parametrize("T,D,shift", [(600, 128, 2.0), (257, 64, 0.0), (128, 128, -3.0)])
def test_gdn_bf16_reduced(dev, oracle, T, D, shift):
    say(f"case: GDN bf16 B=2 T={T} H=4 K=V={D} gate shift {shift} h0 N(0,0.02)")
    d = wl.delta_rule_inputs(B=2, T=T, H=4, K=D, V=D, dtype=torch.bfloat16, seed=11 + T, gate_shift=shift,
                             h0_std=0.02)
    o, ht = sf.gdn_chunk_fwd(cuda(d["q"], dev), cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev),
                             cuda(d["beta"], dev), cuda(d["h0"], dev), output_final_state=True)
    ro, rh = oracle.gdn_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(d["beta"]), f32(d["h0"]))
    check_bf16("reduced", f32(o), ro, f32(ht), rh)


# Launches with more 16-row slices than two per CU (256 CUs on MI355X) take the per-head chain
# kernel (one workgroup per head: its 8 value slices, or in summary mode all its value and
# transition slices); these cases reach it at small sizes, with a ragged last chunk, h0, grouped
# heads and summary mode at both key sizes.
@pytest.mark.parametrize("D,H,HK", [(128, 40, 40), (64, 72, 72), (128, 40, 10)])
def test_gdn_bf16_many_heads(dev, oracle, D, H, HK):
    say(f"case: GDN bf16 B=2 T=200 H={H} HK={HK} K=V={D} (more slices than two per CU) h0 N(0,0.02)")
    d = wl.delta_rule_inputs(B=2, T=200, H=H, HK=HK, K=D, V=D, dtype=torch.bfloat16, seed=D + H + HK,
                             gate_shift=1.0, h0_std=0.02)
    o, ht = sf.gdn_chunk_fwd(cuda(d["q"], dev), cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev),
                             cuda(d["beta"], dev), cuda(d["h0"], dev), output_final_state=True)
    ro, rh = oracle.gdn_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(d["beta"]), f32(d["h0"]))
    check_bf16("many heads", f32(o), ro, f32(ht), rh)


@pytest.mark.parametrize("D,H", [(128, 8), (64, 24)])
def test_gdn_summary_many_rows(dev, oracle, D, H):
    say(f"case: GDN bf16 summary, 8 rows x H={H} K=V={D} (more slices than two per CU), rows with tails")
    d = wl.delta_rule_inputs(B=8, T=200, H=H, K=D, V=D, dtype=torch.bfloat16, seed=77 + D, gate_shift=-5.0,
                             beta_scale=0.3)
    M, E = sf.segment_summary("gdn", cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev), cuda(d["beta"], dev))
    rM, rE = oracle.gdn_summary(f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(d["beta"]))
    assert np.abs(rM).max() > 0.1  # the transition is far from zero here
    eM, eE = rel_rms(f32(M), rM), rel_rms(f32(E), rE)
    say(f"  rel_rms(M)={eM:.3e} rel_rms(S_ext)={eE:.3e}")
    assert eM <= BF16_RTOL and eE <= BF16_RTOL


# Degenerate gates in both bf16 chain kernels (4 heads: one workgroup per 16-row slice; 40 heads:
# one per head): beta = 0 leaves the initial state's pure decay (weak gates, so that it stays
# representable in float32); g = 0 with beta = 1 overwrites along each unit key without decay;
# g = -60 per token underflows every decay factor past the diagonal, and the carried state, to zero
# in float32.
@pytest.mark.parametrize("case", ["beta0", "nodecay", "strongdecay"])
@pytest.mark.parametrize("H", [4, 40])
def test_gdn_bf16_degenerate_gates(dev, oracle, case, H):
    say(f"case: GDN bf16 B=2 T=200 H={H} K=V=128 h0 N(0,0.02), {case}")
    d = wl.delta_rule_inputs(B=2, T=200, H=H, K=128, V=128, dtype=torch.bfloat16, seed=300 + H,
                             gate_shift=-5.0, h0_std=0.02)
    if case == "beta0":
        d["beta"] = torch.zeros_like(d["beta"])
    elif case == "nodecay":
        d["g"] = torch.zeros_like(d["g"])
        d["beta"] = torch.ones_like(d["beta"])
    else:
        d["g"] = torch.full_like(d["g"], -60.0)
    o, ht = sf.gdn_chunk_fwd(cuda(d["q"], dev), cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev),
                             cuda(d["beta"], dev), cuda(d["h0"], dev), output_final_state=True)
    o, ht = f32(o), f32(ht)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    ro, rh = oracle.gdn_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(d["beta"]), f32(d["h0"]))
    check_bf16(case, o, ro, ht, rh)


def test_dense_gdn_full_size(dev, oracle):
    say("case: dense GDN prefill B=2 T=4096 H=16 K=V=128 bf16 (full size, every head vs oracle)")
    w = wl.dense_gdn()
    o, ht = sf.gdn_chunk_fwd(cuda(w.q, dev), cuda(w.k, dev), cuda(w.v, dev), cuda(w.g, dev), cuda(w.beta, dev),
                             cuda(w.h0, dev), scale=w.scale, output_final_state=True)
    torch.cuda.synchronize()
    o, ht = f32(o), f32(ht)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    ro, rh = oracle.gdn_forward(f32(w.q), f32(w.k), f32(w.v), f32(w.g), f32(w.beta), f32(w.h0), scale=w.scale)
    check_bf16("dense, all heads", o, ro, ht, rh)
    check_units("dense per (row, head)", [(f"o b{b} h{h}", o[b, :, h], ro[b, :, h]) for b in range(w.B)
                                           for h in range(w.H)] +
                [(f"ht b{b} h{h}", ht[b, h], rh[b, h]) for b in range(w.B) for h in range(w.H)])


def host_chunk_table(cu, C=64):
    lens = np.diff(cu)
    nch = (lens + C - 1) // C
    off = np.concatenate([[0], np.cumsum(nch)]).astype(np.int32)
    table = [(n, c) for n in range(len(lens)) for c in range(nch[n])]
    return off, table


def test_varlen_gdn_full_size(dev, oracle):
    w = wl.varlen_gdn()
    lens = w.meta["lengths"]
    say(f"case: packed varlen GDN T=32768 H=32 K=V=128 bf16 lengths={lens} (every head and sequence)")
    cu = cuda(w.cu_seqlens, dev)
    h0 = torch.randn(w.N, w.H, w.V, w.K, generator=torch.Generator().manual_seed(5)) * 0.02
    q, k, v, g, beta = (cuda(x, dev) for x in (w.q, w.k, w.v, w.g, w.beta))
    o, ht = sf.gdn_chunk_fwd(q, k, v, g, beta, cuda(h0, dev), cu_seqlens=cu, scale=w.scale, output_final_state=True)
    torch.cuda.synchronize()
    o, ht = f32(o), f32(ht)
    ro, rh = oracle.gdn_forward(f32(w.q), f32(w.k), f32(w.v), f32(w.g), f32(w.beta), f32(h0),
                                cu_seqlens=w.cu_seqlens.numpy(), scale=w.scale)
    end = int(w.cu_seqlens[-1])
    check_bf16("varlen, all heads", o[:, :end], ro[:, :end], ht, rh)
    cu_h = w.cu_seqlens.numpy()
    units = []
    for n, L in enumerate(lens):
        if L == 0:
            # an empty sequence returns its initial state bitwise
            assert np.array_equal(ht[n], f32(h0[n])), "empty sequence must pass its state through"
            continue
        a, b_ = int(cu_h[n]), int(cu_h[n + 1])
        for h in range(w.H):
            units.append((f"o seq{n}(L={L}) h{h}", o[0, a:b_, h], ro[0, a:b_, h]))
            units.append((f"ht seq{n} h{h}", ht[n, h], rh[n, h]))
    check_units("varlen per (sequence, head)", units)


def test_varlen_chunk_table_is_exact(dev):
    # Pre and both bf16 chain kernels index the chunk records of a packed launch through the device chunk
    # table (here H = 64 at K = V = 64: 2304 state slices, the per-head chain)
    say("case: device chunk table vs host table (bit-exact)")
    lens = [0, 5, 64, 0, 130, 1, 63, 700, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1]) + 37
    N, H = len(lens), 64
    d = wl.delta_rule_inputs(B=1, T=T, H=H, K=64, V=64, dtype=torch.bfloat16, seed=3)
    L = sf.lib()
    nbytes = L.sf_gdn_chunk_fwd_workspace(sf.SF_BF16, 1, T, H, 64, 64, N, 1)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    q, k, v, g, beta = (cuda(d[x], dev) for x in ("q", "k", "v", "g", "beta"))
    out = torch.empty_like(v)
    cu_d = torch.from_numpy(cu).to(dev)
    import ctypes
    st = L.sf_gdn_chunk_fwd(sf.SF_BF16, *(ctypes.c_void_p(t.data_ptr()) for t in (q, k, v, g, beta)), None,
                            ctypes.c_void_p(cu_d.data_ptr()), N, 1, T, H, H, 64, 64, 0.125,
                            ctypes.c_void_p(out.data_ptr()), None, ctypes.c_void_p(ws.data_ptr()), nbytes,
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.sf_last_error()
    torch.cuda.synchronize()
    cap = (T + 63) // 64 + N
    raw = ws.cpu().numpy()
    off_dev = raw[:4 * (N + 1)].view(np.int32)
    tab_base = (4 * (N + 1) + 255) // 256 * 256
    tab_dev = raw[tab_base:tab_base + 8 * cap].view(np.int32).reshape(cap, 2)
    off, table = host_chunk_table(cu)
    assert np.array_equal(off_dev, off)
    assert [tuple(x) for x in tab_dev[:len(table)]] == table
    assert (tab_dev[len(table):, 0] == -1).all()


# Packed sequences against each sequence alone, bit for bit. With H = 32, K = V = 128 and the packed
# workload's own nine lengths, the packed launch (2304 16-row slices) runs the per-head chain kernel while
# each sequence alone (256 slices) runs the per-slice kernel; both read the same Pre records and take every
# per-chunk step from the same code. H = 4 runs the per-slice kernel on both sides, H = 72 the per-head
# kernel on both.
@pytest.mark.parametrize("case", ["packed-workload-shape", "H4", "H72"])
def test_packed_equals_alone_bitwise(dev, case):
    if case == "packed-workload-shape":
        w = wl.varlen_gdn()
        lens, H = w.meta["lengths"], w.H
        cu = w.cu_seqlens.numpy()
        T = w.T
        d = dict(q=w.q, k=w.k, v=w.v, g=w.g, beta=w.beta)
    else:
        lens = [130, 0, 64, 7, 300]
        H = 4 if case == "H4" else 72
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(cu[-1]) + 20
        d = wl.delta_rule_inputs(B=1, T=T, H=H, K=128, V=128, dtype=torch.bfloat16, seed=21, gate_shift=-1.0)
    say(f"case: packed sequences equal separate dense calls bitwise, {case}: H={H} K=V=128 lengths {list(lens)}")
    h0 = torch.randn(len(lens), H, 128, 128, generator=torch.Generator().manual_seed(1)) * 0.1
    q, k, v, g, beta = (cuda(d[x], dev) for x in ("q", "k", "v", "g", "beta"))
    h0d = cuda(h0, dev)
    o, ht = sf.gdn_chunk_fwd(q, k, v, g, beta, h0d, cu_seqlens=torch.from_numpy(cu).to(dev),
                             output_final_state=True)
    for n, L in enumerate(lens):
        a, b_ = int(cu[n]), int(cu[n + 1])
        if L == 0:
            assert torch.equal(ht[n], h0d[n])
            continue
        sl = lambda x: x[:, a:b_].contiguous()
        o1, h1 = sf.gdn_chunk_fwd(sl(q), sl(k), sl(v), sl(g), sl(beta), h0d[n:n + 1].contiguous(),
                                  output_final_state=True)
        assert torch.equal(o[:, a:b_], o1), f"sequence {n} (length {L}) differs from its separate run"
        assert torch.equal(ht[n], h1[0]), f"sequence {n} final state differs from its separate run"
    if case == "packed-workload-shape":
        return
    # GLA: same packing invariant
    o2, h2 = sf.gla_chunk_fwd(q, k, v, g, h0d, cu_seqlens=torch.from_numpy(cu).to(dev), chunk=64,
                              output_final_state=True)
    for n, L in enumerate(lens):
        a, b_ = int(cu[n]), int(cu[n + 1])
        if L == 0:
            assert torch.equal(h2[n], h0d[n])
            continue
        sl = lambda x: x[:, a:b_].contiguous()
        o3, h3 = sf.gla_chunk_fwd(sl(q), sl(k), sl(v), sl(g), h0d[n:n + 1].contiguous(), chunk=64,
                                  output_final_state=True)
        assert torch.equal(o2[:, a:b_], o3)
        assert torch.equal(h2[n], h3[0])


def test_rows_past_terminal_offset_are_not_written(dev):
    say("case: output rows past cu_seqlens[-1] keep their contents")
    import ctypes
    lens = [70, 30]
    cu = torch.tensor([0, 70, 100], dtype=torch.int32)
    T, H = 160, 2
    d = wl.delta_rule_inputs(B=1, T=T, H=H, K=64, V=64, dtype=torch.bfloat16, seed=4)
    q, k, v, g, beta = (cuda(d[x], dev) for x in ("q", "k", "v", "g", "beta"))
    for kind in ("gdn", "gla"):
        out = torch.full_like(v, 3.0)
        L = sf.lib()
        cu_d = cu.to(dev)
        P = lambda t: ctypes.c_void_p(t.data_ptr())
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if kind == "gdn":
            nb = L.sf_gdn_chunk_fwd_workspace(sf.SF_BF16, 1, T, H, 64, 64, 2, 1)
            ws = torch.empty(nb, dtype=torch.uint8, device=dev)
            st = L.sf_gdn_chunk_fwd(sf.SF_BF16, P(q), P(k), P(v), P(g), P(beta), None, P(cu_d), 2, 1, T, H, H, 64, 64,
                                    0.125, P(out), None, P(ws), nb, s)
        else:
            st = L.sf_gla_chunk_fwd(sf.SF_BF16, P(q), P(k), P(v), P(g), None, P(cu_d), 2, 1, T, H, H, 64, 64, 64, 1.0,
                                    P(out), None, s)
        assert st == 0
        torch.cuda.synchronize()
        assert (out[:, 100:] == 3.0).all()
        assert not (out[:, :100] == 3.0).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_resume_from_final_state(dev, oracle, dtype):
    say(f"case: {dtype} one call on [0,T) vs [0,t) then [t,T) with the state passed (t a multiple of 64)")
    d = wl.delta_rule_inputs(B=2, T=448, H=2, K=128, V=128, dtype=dtype, seed=9, gate_shift=-2.0, h0_std=0.1)
    x = {n: cuda(d[n], dev) for n in ("q", "k", "v", "g", "beta", "h0")}
    o, ht = sf.gdn_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], output_final_state=True)
    t = 192
    a = {n: x[n][:, :t].contiguous() for n in ("q", "k", "v", "g", "beta")}
    b = {n: x[n][:, t:].contiguous() for n in ("q", "k", "v", "g", "beta")}
    o1, h1 = sf.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], x["h0"], output_final_state=True)
    o2, h2 = sf.gdn_chunk_fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], h1, output_final_state=True)
    # each chunk's factors depend on the chunk alone and the state is carried in float32, so a split at a
    # chunk boundary changes no bit
    assert torch.equal(o[:, :t], o1) and torch.equal(o[:, t:], o2) and torch.equal(ht, h2)


# ---------------------------------------------------------------------------
# Summaries and the scan
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.bfloat16, 128), (torch.bfloat16, 64)])
def test_gdn_summary_vs_oracle(dev, oracle, dtype, D):
    say(f"case: GDN summary {dtype} K=V={D}, rows with tails")
    R, L = 3, 200
    d = wl.delta_rule_inputs(B=R, T=L, H=2, K=D, V=D, dtype=dtype, seed=D + 3, gate_shift=-5.0,
                             beta_scale=0.3)
    M, E = sf.segment_summary("gdn", cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev), cuda(d["beta"], dev))
    rM, rE = oracle.gdn_summary(f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(d["beta"]))
    assert np.abs(rM).max() > 0.1  # the transition is far from zero here
    if dtype == torch.float32:
        eM, eE = maxabs(f32(M), rM), maxabs(f32(E), rE)
        say(f"  max|M-ref|={eM:.3e} max|S_ext-ref|={eE:.3e}")
        assert eM <= FP32_ATOL and eE <= FP32_ATOL
    else:
        eM, eE = rel_rms(f32(M), rM), rel_rms(f32(E), rE)
        say(f"  rel_rms(M)={eM:.3e} rel_rms(S_ext)={eE:.3e}")
        assert eM <= BF16_RTOL and eE <= BF16_RTOL


@pytest.mark.parametrize("dtype,chunk", [(torch.float32, 64), (torch.bfloat16, 128), (torch.bfloat16, 64)])
def test_gla_summary_vs_oracle(dev, oracle, dtype, chunk):
    say(f"case: GLA summary {dtype} chunk {chunk}")
    d = wl.scalar_gate_inputs(B=3, T=300, H=4, HK=2, K=128, V=64, dtype=dtype, seed=chunk)
    # slow the gates so that a_block = exp(sum g) stays in the float32 range (sum g ~ -3)
    d["g"] = d["g"] * 0.02
    a, E = sf.segment_summary("gla", cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev), chunk=chunk)
    ra, rE = oracle.gla_summary(f32(d["k"]), f32(d["v"]), f32(d["g"]))
    ea = float(np.max(np.abs(f32(a) - ra) / ra))
    say(f"  max rel|a-ref|={ea:.3e} rel_rms(S_ext)={rel_rms(f32(E), rE):.3e}")
    assert ra.min() > 1e-6 and ea <= 1e-4
    if dtype == torch.float32:
        assert maxabs(f32(E), rE) <= FP32_ATOL * max(1.0, np.abs(rE).max())
    else:
        assert rel_rms(f32(E), rE) <= BF16_RTOL


@pytest.mark.parametrize("kind,D", [("gdn", 128), ("gdn", 64), ("gla", 128)])
def test_state_scan_vs_oracle(dev, oracle, kind, D):
    say(f"case: state scan {kind} K=V={D}")
    B, n_seg, H = 2, 5, 3
    rng = np.random.default_rng(D)
    if kind == "gdn":
        M = (rng.standard_normal((B * n_seg, H, D, D)) / np.sqrt(D)).astype(np.float32)
    else:
        M = rng.uniform(0.2, 1.0, (B * n_seg, H)).astype(np.float32)
    E = rng.standard_normal((B * n_seg, H, D, D)).astype(np.float32)
    h0 = rng.standard_normal((B, H, D, D)).astype(np.float32)
    S_in, S_f = sf.state_scan(kind, torch.from_numpy(M).to(dev), torch.from_numpy(E).to(dev),
                              torch.from_numpy(h0).to(dev), B=B, n_seg=n_seg)
    rS, rF = oracle.state_scan(kind, M, E, h0, B=B, n_seg=n_seg)
    e1, e2 = maxabs(f32(S_in), rS), maxabs(f32(S_f), rF)
    say(f"  max|S_in-ref|={e1:.3e} max|S_final-ref|={e2:.3e} (|ref| max {np.abs(rF).max():.2f})")
    assert np.array_equal(f32(S_in)[0::n_seg], h0)  # exclusive: first segment starts at h0 exactly
    assert e1 <= 1e-4 * max(1.0, np.abs(rS).max()) and e2 <= 1e-4 * max(1.0, np.abs(rF).max())


def test_segmented_gdn_nonzero_transitions(dev, oracle):
    say("case: segmented GDN B=1 T=4096 H=4 K=V=64, 16 segments of 256, slow gates (M far from 0)")
    d = wl.delta_rule_inputs(B=1, T=4096, H=4, K=64, V=64, dtype=torch.bfloat16, seed=77, gate_shift=-6.0,
                             beta_scale=0.1, h0_std=0.1)
    x = {n: cuda(d[n], dev) for n in ("q", "k", "v", "g", "beta", "h0")}
    o, hf = sf.segmented_gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], 16, x["h0"], output_final_state=True)
    ro, rh = oracle.gdn_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(d["beta"]), f32(d["h0"]))
    check_bf16("segmented vs unsegmented oracle", f32(o), ro, f32(hf), rh)
    M, _ = sf.segment_summary("gdn", *(sf.segment_view(x[n], 16) for n in ("k", "v", "g", "beta")))
    diag = np.einsum("shii->shi", f32(M))
    assert diag.mean() > 0.1  # the transitions are far from zero, so the scan matters


# ---------------------------------------------------------------------------
# Scalar-gated linear attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,chunk,T,HK", [(torch.float32, 64, 200, 2), (torch.bfloat16, 64, 129, 1),
                                              (torch.bfloat16, 128, 300, 2), (torch.bfloat16, 128, 1, 4)])
def test_gla_vs_oracle(dev, oracle, dtype, chunk, T, HK):
    say(f"case: GLA {dtype} chunk {chunk} T={T} H=4 HK={HK} K=128 V=64 with h0")
    d = wl.scalar_gate_inputs(B=2, T=T, H=4, HK=HK, K=128, V=64, dtype=dtype, seed=T)
    h0 = (torch.randn(2, 4, 64, 128, generator=torch.Generator().manual_seed(T))).float()
    o, ht = sf.gla_chunk_fwd(cuda(d["q"], dev), cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev),
                             cuda(h0, dev), chunk=chunk, scale=0.5, output_final_state=True)
    ro, rh = oracle.gla_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(h0), scale=0.5)
    if dtype == torch.float32:
        # unnormalised q/k: outputs reach ~1e2, so the float32 bound scales with them
        eo, eh = maxabs(f32(o), ro), maxabs(f32(ht), rh)
        so, sh = max(1.0, np.abs(ro).max()), max(1.0, np.abs(rh).max())
        say(f"  max|o-ref|/max(1,|ref|)={eo / so:.3e} max|ht-ref|/max(1,|ref|)={eh / sh:.3e}")
        assert eo <= FP32_ATOL * so and eh <= FP32_ATOL * sh
    else:
        check_bf16("gla", f32(o), ro, f32(ht), rh)


def test_segmented_gla_nonzero_transitions(dev, oracle):
    """Segmented scalar gate with a_block far from zero: the gates are slowed so that each segment's gate
    sum is about -2 (a_block ~ 0.1), so the scan's a * S_in term carries real weight into every segment."""
    say("case: segmented GLA B=2 T=4096 H=8 HK=2 K=128 V=64 chunk 128, 8 segments of 512, a_block ~ 0.1")
    d = wl.scalar_gate_inputs(B=2, T=4096, H=8, HK=2, K=128, V=64, seed=91)
    g = d["g"]
    seg_sums = g.view(2, 8, 512, 8).sum(2)
    d["g"] = (g * (-2.0 / float(seg_sums.median()))).float().contiguous()
    h0 = (torch.randn(2, 8, 64, 128, generator=torch.Generator().manual_seed(91)) * 0.1).float()
    x = {n: cuda(d[n], dev) for n in ("q", "k", "v", "g")}
    o, hf = sf.segmented_gla_fwd(x["q"], x["k"], x["v"], x["g"], 8, cuda(h0, dev), scale=0.1, chunk=128,
                                 output_final_state=True)
    a, _ = sf.segment_summary("gla", sf.segment_view(x["k"], 8), sf.segment_view(x["v"], 8),
                              sf.segment_view(x["g"], 8), chunk=128)
    a = f32(a)
    say(f"  a_block range [{a.min():.3f}, {a.max():.3f}]")
    assert a.min() > 1e-3 and np.median(a) > 0.05  # the scan's a * S_in term is far from zero
    ro, rh = oracle.gla_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(h0), scale=0.1)
    check_bf16("segmented vs unsegmented oracle", f32(o), ro, f32(hf), rh)
    o_ = f32(o)
    check_units("per (row, segment, head)", [(f"o b{b} seg{j} h{h}", o_[b, 512 * j:512 * (j + 1), h],
                                              ro[b, 512 * j:512 * (j + 1), h])
                                             for b in range(2) for j in range(8) for h in range(8)])


# bf16 scalar-gate shapes the ABI accepts, each against the oracle: K, V in {64, 128}, chunk 64 and 128,
# grouped heads, a ragged last chunk and an initial state.
@pytest.mark.parametrize("K,V,chunk", [(64, 64, 64), (64, 64, 128), (128, 128, 64), (128, 128, 128),
                                       (64, 128, 128), (128, 64, 64), (64, 128, 64)])
def test_gla_bf16_shapes_vs_oracle(dev, oracle, K, V, chunk):
    say(f"case: GLA bf16 K={K} V={V} chunk {chunk} B=2 T=300 H=4 HK=2 with h0")
    d = wl.scalar_gate_inputs(B=2, T=300, H=4, HK=2, K=K, V=V, seed=K + V + chunk)
    h0 = (torch.randn(2, 4, V, K, generator=torch.Generator().manual_seed(K + V)) * 0.3).float()
    o, ht = sf.gla_chunk_fwd(cuda(d["q"], dev), cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev),
                             cuda(h0, dev), chunk=chunk, scale=0.3, output_final_state=True)
    ro, rh = oracle.gla_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(h0), scale=0.3)
    check_bf16(f"gla K={K} V={V} chunk {chunk}", f32(o), ro, f32(ht), rh)


def test_document_aligned_split_is_bitwise(dev):
    """A packed stream cut at a document boundary into two calls gives, bit for bit, the results of the
    single call (attention-gym "Context Parallelism", document-aligned fragments): each document's
    arithmetic does not depend on which others share its launch. Delta rule and scalar gate."""
    lens = [130, 0, 64, 7, 300, 91, 1]
    cut = 3   # documents [0, 3) and [3, 7)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    H = 32
    say(f"case: document-aligned split, lengths {lens}, cut before document {cut}, H={H} K=V=128")
    d = wl.delta_rule_inputs(B=1, T=T, H=H, K=128, V=128, dtype=torch.bfloat16, seed=23, gate_shift=-1.0)
    h0 = (torch.randn(len(lens), H, 128, 128, generator=torch.Generator().manual_seed(2)) * 0.1).float()
    x = {n: cuda(d[n], dev) for n in ("q", "k", "v", "g", "beta")}
    h0d = cuda(h0, dev)
    t = int(cu[cut])
    part = lambda a, b: {n: x[n][:, a:b].contiguous() for n in x}
    cu_a = torch.from_numpy(cu[:cut + 1]).to(dev)
    cu_b = torch.from_numpy(cu[cut:] - t).to(dev)
    for kind in ("gdn", "gla"):
        if kind == "gdn":
            run = lambda y, hh, c: sf.gdn_chunk_fwd(y["q"], y["k"], y["v"], y["g"], y["beta"], hh, cu_seqlens=c,
                                                    output_final_state=True)
        else:
            run = lambda y, hh, c: sf.gla_chunk_fwd(y["q"], y["k"], y["v"], y["g"], hh, cu_seqlens=c, chunk=64,
                                                    scale=0.2, output_final_state=True)
        o, ht = run(x, h0d, torch.from_numpy(cu).to(dev))
        oa, ha = run(part(0, t), h0d[:cut].contiguous(), cu_a)
        ob, hb = run(part(t, T), h0d[cut:].contiguous(), cu_b)
        assert torch.equal(o[:, :t], oa) and torch.equal(o[:, t:T], ob), kind
        assert torch.equal(ht[:cut], ha) and torch.equal(ht[cut:], hb), kind


# Degenerate scalar gates: g = 0 is causal linear attention (no decay, the state grows), g = -60
# per token underflows every decay past the diagonal and the carried state.
@pytest.mark.parametrize("case", ["nodecay", "strongdecay"])
def test_gla_bf16_degenerate_gates(dev, oracle, case):
    say(f"case: GLA bf16 chunk 128 T=300 H=4 HK=2 K=128 V=64 with h0, {case}")
    d = wl.scalar_gate_inputs(B=2, T=300, H=4, HK=2, K=128, V=64, dtype=torch.bfloat16, seed=31)
    d["g"] = torch.zeros_like(d["g"]) if case == "nodecay" else torch.full_like(d["g"], -60.0)
    h0 = (torch.randn(2, 4, 64, 128, generator=torch.Generator().manual_seed(31))).float()
    o, ht = sf.gla_chunk_fwd(cuda(d["q"], dev), cuda(d["k"], dev), cuda(d["v"], dev), cuda(d["g"], dev),
                             cuda(h0, dev), chunk=128, scale=0.05, output_final_state=True)
    o, ht = f32(o), f32(ht)
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    ro, rh = oracle.gla_forward(f32(d["q"]), f32(d["k"]), f32(d["v"]), f32(d["g"]), f32(h0), scale=0.05)
    check_bf16(case, o, ro, ht, rh)


def test_ssd_gla_full_size_segmented(dev, oracle):
    say("case: SSD-shaped GLA B=2 T=16384 H=64 HK=8 K=128 V=64 chunk 128, 8 segments per row (full size, all heads)")
    w = wl.ssd_gla()
    x = {n: cuda(getattr(w, n), dev) for n in ("q", "k", "v", "g")}
    o, hf = sf.segmented_gla_fwd(x["q"], x["k"], x["v"], x["g"], w.n_seg, scale=w.scale, chunk=w.chunk,
                                 output_final_state=True)
    ou, hu = sf.gla_chunk_fwd(x["q"], x["k"], x["v"], x["g"], scale=w.scale, chunk=w.chunk,
                              output_final_state=True)
    torch.cuda.synchronize()
    ro, rh = oracle.gla_forward(f32(w.q), f32(w.k), f32(w.v), f32(w.g), scale=w.scale)
    o, hf, ou, hu = f32(o), f32(hf), f32(ou), f32(hu)
    check_bf16("segmented", o, ro, hf, rh)
    check_bf16("unsegmented", ou, ro, hu, rh)
    check_units("segmented per (row, head)", [(f"o b{b} h{h}", o[b, :, h], ro[b, :, h]) for b in range(w.B)
                                               for h in range(w.H)])


def test_long_gdn_full_size_segmented(dev, oracle):
    say("case: long GDN B=1 T=262144 H=16 K=V=128 bf16, 16 segments of 16384 (full size; every head vs oracle)")
    w = wl.long_gdn()
    x = {n: cuda(getattr(w, n), dev) for n in ("q", "k", "v", "g", "beta")}
    o, hf = sf.segmented_gdn_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], w.n_seg, scale=w.scale,
                                 output_final_state=True)
    torch.cuda.synchronize()
    o, hf = f32(o), f32(hf)
    say("  GPU done; oracle on all 16 heads over 262144 tokens")
    ro, rh = oracle.gdn_forward(f32(w.q), f32(w.k), f32(w.v), f32(w.g), f32(w.beta), scale=w.scale)
    check_bf16("segmented, all heads", o, ro, hf, rh)
    L = w.T // w.n_seg
    check_units("segmented per (segment, head)", [(f"o seg{j} h{h}", o[0, j * L:(j + 1) * L, h],
                                                   ro[0, j * L:(j + 1) * L, h])
                                                  for j in range(w.n_seg) for h in range(w.H)])

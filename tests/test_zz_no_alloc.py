"""The chunk forward entry point that allocates nothing (sf_gdn_chunk_fwd_noalloc), through the C ABI,
against sf_gdn_chunk_fwd on the same inputs: two calls in a row, the second with a smaller (packed)
input, so the static scratch holds the first call's contents when the second starts. Both entry points
run the same kernels on the same arithmetic, so their results must agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import chunked_linear_recurrence_amd as sf
import workloads as wl

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_both(d, dev, cu=None, N=None):
    L = sf.lib()
    q, k, v, g, beta = (d[n].to(dev).contiguous() for n in ("q", "k", "v", "g", "beta"))
    h0 = None if d.get("h0") is None else d["h0"].to(dev).contiguous()
    B, T, HK, K = q.shape
    H, V = v.shape[2], v.shape[3]
    N = B if cu is None else cu.numel() - 1
    cu_d = None if cu is None else cu.to(dev)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # the entry point with a caller workspace
    o1 = torch.full_like(v, 7.0)
    h1 = torch.full((N, H, V, K), 7.0, dtype=torch.float32, device=dev)
    nb = L.sf_gdn_chunk_fwd_workspace(sf.SF_BF16, B, T, H, K, V, N, int(cu is not None))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    st = L.sf_gdn_chunk_fwd(sf.SF_BF16, P(q), P(k), P(v), P(g), P(beta), P(h0), P(cu_d), N, B, T, H, HK, K, V,
                            0.125, P(o1), P(h1), P(ws), nb, s)
    assert st == 0, L.sf_last_error()
    # the same call with no workspace argument (static scratch)
    o2 = torch.full_like(v, 7.0)
    h2 = torch.full((N, H, V, K), 7.0, dtype=torch.float32, device=dev)
    st = L.sf_gdn_chunk_fwd_noalloc(sf.SF_BF16, P(q), P(k), P(v), P(g), P(beta), P(h0), P(cu_d), N, B, T, H, HK,
                                    K, V, 0.125, P(o2), P(h2), s)
    assert st == 0, L.sf_last_error()
    torch.cuda.synchronize()
    return o1, h1, o2, h2


def test_noalloc_matches_workspace_entry_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    L = sf.lib()
    assert L.sf_static_scratch_bytes() == 64 << 20
    say("no-alloc call 1: dense B=2 T=4096 H=16 K=V=128 bf16 with h0 (52 MB of scratch)")
    d = wl.delta_rule_inputs(B=2, T=4096, H=16, K=128, V=128, dtype=torch.bfloat16, seed=61, gate_shift=2.0,
                             h0_std=0.02)
    o1, h1, o2, h2 = run_both(d, dev)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    say("no-alloc call 2: packed, 4 sequences, H=4 K=V=64 (smaller, chunk table in the scratch)")
    lens = [70, 0, 130, 5]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    d = wl.delta_rule_inputs(B=1, T=int(cu[-1]) + 9, H=4, K=64, V=64, dtype=torch.bfloat16, seed=62,
                             h0_std=0.1, N=len(lens))
    o1, h1, o2, h2 = run_both(d, dev, cu=cu)
    end = int(cu[-1])
    assert torch.equal(o1[:, :end], o2[:, :end]) and torch.equal(h1, h2)
    assert (o2[:, end:] == 7.0).all()  # rows past the terminal offset are not written
    # sizes past the static scratch are rejected before anything is enqueued
    big = L.sf_gdn_chunk_fwd_workspace(sf.SF_BF16, 1, 1 << 18, 16, 128, 128, 1, 0)
    assert big > (64 << 20)
    F = ctypes.c_void_p(0x1000)
    st = L.sf_gdn_chunk_fwd_noalloc(sf.SF_BF16, F, F, F, F, F, None, None, 1, 1, 1 << 18, 16, 16, 128, 128, 0.1, F,
                                    None, None)
    assert st == sf.SF_ERR_WORKSPACE and b"static" in L.sf_last_error()

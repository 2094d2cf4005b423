"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes its workspaces, and rejects invalid arguments on the
host before anything is enqueued (attention-gym "Linear Attention": unsupported
choices fail instead of falling back)."""
import ctypes
import os
import re

import pytest

import chunked_linear_recurrence_amd as sf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sf.h")

FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sf.LIB_PATH):
        from chunked_linear_recurrence_amd import build
        build.build(verbose=False)
    return sf.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sf_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("sf_gdn_chunk_fwd", "sf_segment_summary", "sf_state_scan", "sf_gla_chunk_fwd"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"{n} is declared in sf.h but not exported"
    assert set(names) == set(sf.EXPORTED)


def test_version(L):
    assert sf.version().startswith("sf ") and "gfx950" in sf.version()


def test_workspace_sizes(L):
    rec = 6 * 1024 + 1024  # bf16 factor record: T diag(beta) fragments, coefficients
    dense = L.sf_gdn_chunk_fwd_workspace(sf.SF_BF16, 2, 4096, 16, 128, 128, 2, 0)
    assert dense == 2 * 64 * 16 * rec
    # packed: chunk offsets (N+1 ints) and table (cap int2), each 256-aligned, then factors
    N, T, H = 9, 32768, 32
    cap = (T + 63) // 64 + N
    al = lambda x: (x + 255) // 256 * 256
    packed = L.sf_gdn_chunk_fwd_workspace(sf.SF_BF16, 1, T, H, 128, 128, N, 1)
    assert packed == al(4 * (N + 1)) + al(8 * cap) + al(cap * H * rec)
    assert L.sf_gdn_chunk_fwd_workspace(sf.SF_F32, 1, 256, 2, 64, 64, 1, 0) == 4 * 2 * (2 * 64 * 64 * 4 + 1024)
    assert L.sf_segment_summary_workspace(sf.SF_KIND_GLA, sf.SF_BF16, 16, 2048, 64, 128, 64, 128) == 0
    assert L.sf_gdn_chunk_fwd_workspace(7, 1, 1, 1, 64, 64, 1, 0) == 0


def test_segmented_workspace_size(L):
    # per segment row: the Pre records, then M [rows, H, K, K], S_ext and S_in [rows, H, V, K], float32,
    # each 256-aligned
    rec = 6 * 1024 + 1024
    al = lambda x: (x + 255) // 256 * 256
    B, n_seg, T, H, K = 1, 16, 262144, 16, 128
    rows, L_seg = B * n_seg, T // n_seg
    want = al(rows * (L_seg // 64) * H * rec) + al(4 * rows * H * K * K) + 2 * al(4 * rows * H * K * K)
    assert L.sf_gdn_segmented_fwd_workspace(sf.SF_BF16, B, n_seg, T, H, K, K) == want
    assert L.sf_gdn_segmented_fwd_workspace(sf.SF_BF16, 1, 3, 1000, 4, 64, 64) == 0  # T not a multiple of n_seg


@pytest.mark.parametrize("kw,status,msg", [
    (dict(T=1000, n_seg=8), sf.SF_ERR_INVALID, "multiple of the chunk"),
    (dict(T=999, n_seg=8), sf.SF_ERR_INVALID, "multiple of n_seg"),
    (dict(n_seg=0), sf.SF_ERR_INVALID, "multiple of n_seg"),
    (dict(q=None), sf.SF_ERR_INVALID, "NULL"),
    (dict(K=96, V=96), sf.SF_ERR_UNSUPPORTED, "K == V"),
    (dict(wsb=16), sf.SF_ERR_WORKSPACE, "workspace"),
])
def test_segmented_rejects_before_enqueue(L, kw, status, msg):
    a = dict(dt=sf.SF_BF16, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, B=1, n_seg=4, T=1024, H=4, HK=4,
             K=128, V=128, scale=0.1, out=FAKE, ht=None, ws=FAKE * 256, wsb=1 << 40, s=None)
    a.update(kw)
    st = L.sf_gdn_segmented_fwd(a["dt"], a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["B"], a["n_seg"],
                                a["T"], a["H"], a["HK"], a["K"], a["V"], a["scale"], a["out"], a["ht"], a["ws"],
                                a["wsb"], a["s"])
    assert st == status and msg in L.sf_last_error().decode()


def gdn_call(L, **kw):
    a = dict(dt=sf.SF_BF16, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, N=2, B=2, T=64,
             H=4, HK=4, K=128, V=128, scale=0.1, out=FAKE, ht=None, ws=FAKE * 256, wsb=1 << 40, s=None)
    a.update(kw)
    st = L.sf_gdn_chunk_fwd(a["dt"], a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"], a["N"], a["B"],
                            a["T"], a["H"], a["HK"], a["K"], a["V"], a["scale"], a["out"], a["ht"], a["ws"],
                            a["wsb"], a["s"])
    return st, L.sf_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(HK=3), sf.SF_ERR_INVALID, "divide"),
    (dict(q=None), sf.SF_ERR_INVALID, "NULL"),
    (dict(beta=None), sf.SF_ERR_INVALID, "NULL"),
    (dict(dt=5), sf.SF_ERR_INVALID, "dtype"),
    (dict(N=3), sf.SF_ERR_INVALID, "N (3) must equal B"),
    (dict(cu=FAKE, B=2), sf.SF_ERR_INVALID, "batch-one"),
    (dict(K=96, V=96), sf.SF_ERR_UNSUPPORTED, "K == V"),
    (dict(K=128, V=64), sf.SF_ERR_UNSUPPORTED, "K == V"),
    (dict(wsb=16), sf.SF_ERR_WORKSPACE, "smaller"),
    (dict(ws=None), sf.SF_ERR_WORKSPACE, "smaller"),
    (dict(ws=FAKE * 256 + 8), sf.SF_ERR_INVALID, "aligned"),
    (dict(T=1 << 20, H=128, HK=128, B=2, N=2), sf.SF_ERR_UNSUPPORTED, "2^31"),
    (dict(H=-1), sf.SF_ERR_INVALID, "positive"),
    (dict(q=FAKE + 2), sf.SF_ERR_INVALID, "16-byte aligned"),
    (dict(out=FAKE + 8), sf.SF_ERR_INVALID, "16-byte aligned"),
])
def test_gdn_rejects_invalid_arguments(L, kw, status, msg):
    st, err = gdn_call(L, **kw)
    assert st == status, err
    assert msg in err


def test_gla_rejects_invalid_arguments(L):
    call = lambda dt=sf.SF_BF16, K=128, V=64, chunk=128, H=64, HK=8: L.sf_gla_chunk_fwd(
        dt, FAKE, FAKE, FAKE, FAKE, None, None, 2, 2, 128, H, HK, K, V, chunk, 1.0, FAKE, None, None)
    assert call(chunk=32) == sf.SF_ERR_UNSUPPORTED
    assert call(dt=sf.SF_F32, chunk=128) == sf.SF_ERR_UNSUPPORTED
    assert call(K=96) == sf.SF_ERR_UNSUPPORTED
    assert call(HK=7) == sf.SF_ERR_INVALID


def test_summary_and_scan_reject_invalid_arguments(L):
    st = L.sf_segment_summary(sf.SF_KIND_GDN, sf.SF_BF16, FAKE, FAKE, FAKE, None, 16, 256, 4, 4, 128, 128, 64,
                              FAKE, FAKE, FAKE * 256, 1 << 40, None)
    assert st == sf.SF_ERR_INVALID and "beta" in L.sf_last_error().decode()
    st = L.sf_segment_summary(sf.SF_KIND_GDN, sf.SF_BF16, FAKE, FAKE, FAKE, FAKE, 16, 256, 4, 4, 128, 128, 128,
                              FAKE, FAKE, FAKE * 256, 1 << 40, None)
    assert st == sf.SF_ERR_UNSUPPORTED
    st = L.sf_segment_summary(9, sf.SF_BF16, FAKE, FAKE, FAKE, FAKE, 16, 256, 4, 4, 128, 128, 64,
                              FAKE, FAKE, FAKE * 256, 1 << 40, None)
    assert st == sf.SF_ERR_INVALID
    st = L.sf_state_scan(sf.SF_KIND_GDN, FAKE, FAKE, None, 1, 4, 4, 96, 128, FAKE, None, None)
    assert st == sf.SF_ERR_UNSUPPORTED
    st = L.sf_state_scan(sf.SF_KIND_GDN, None, FAKE, None, 1, 4, 4, 128, 128, FAKE, None, None)
    assert st == sf.SF_ERR_INVALID
    st = L.sf_state_scan(3, FAKE, FAKE, None, 1, 4, 4, 128, 128, FAKE, None, None)
    assert st == sf.SF_ERR_INVALID


def test_decode_rejects_invalid_arguments(L):
    def call(dt=sf.SF_BF16, pool_dt=sf.SF_F32, B=4, H=8, HK=4, K=128, V=128, slots=9, stride=None, pool=FAKE * 16,
             qkv=FAKE * 16, idx=FAKE):
        stride = H * V * K if stride is None else stride
        st = L.sf_gdn_decode(dt, qkv, FAKE, FAKE, FAKE, FAKE, pool, pool_dt, slots, stride, idx, None, B, H, HK, K, V,
                             1.0, FAKE, None)
        return st, L.sf_last_error().decode()
    assert call(K=96)[0] == sf.SF_ERR_UNSUPPORTED
    assert call(K=512)[0] == sf.SF_ERR_UNSUPPORTED
    assert call(V=72)[0] == sf.SF_ERR_UNSUPPORTED
    assert call(HK=3)[0] == sf.SF_ERR_INVALID
    assert call(dt=5)[0] == sf.SF_ERR_INVALID
    assert call(pool_dt=5)[0] == sf.SF_ERR_INVALID
    st, err = call(stride=8 * 128 * 128 - 4)
    assert st == sf.SF_ERR_INVALID and "slot_stride" in err
    assert call(stride=8 * 128 * 128 + 2)[0] == sf.SF_ERR_INVALID
    st, err = call(pool=FAKE * 16 + 8)
    assert st == sf.SF_ERR_INVALID and "aligned" in err
    st, err = call(idx=None)
    assert st == sf.SF_ERR_INVALID and "NULL" in err
    assert call(B=0, idx=None)[0] == sf.SF_OK  # nothing to do, nothing enqueued


def test_recurrent_rejects_invalid_arguments(L):
    def call(K=128, V=128, H=4, HK=2, h0=None, ht=None, pool=None, idx=None, fresh=None, stride=0, B=2, N=2, cu=None,
             dt=sf.SF_BF16, q=FAKE):
        st = L.sf_gdn_recurrent_fwd(dt, q, FAKE, FAKE, FAKE, FAKE, h0, cu, N, B, 16, H, HK, K, V, 1.0, FAKE, ht, pool,
                                    sf.SF_F32, 9, stride, idx, fresh, None)
        return st, L.sf_last_error().decode()
    assert call(K=96)[0] == sf.SF_ERR_UNSUPPORTED
    assert call(V=48)[0] == sf.SF_ERR_UNSUPPORTED
    assert call(HK=3)[0] == sf.SF_ERR_INVALID
    assert call(N=3)[0] == sf.SF_ERR_INVALID            # N != B without cu_seqlens
    st, err = call(idx=FAKE, h0=FAKE * 16, pool=FAKE * 16, stride=4 * 128 * 128)
    assert st == sf.SF_ERR_INVALID and "NULL" in err    # h0 with a pool
    st, err = call(idx=FAKE, pool=FAKE * 16, stride=4 * 128 * 128 - 4)
    assert st == sf.SF_ERR_INVALID and "slot_stride" in err
    st, err = call(idx=FAKE, pool=None, stride=4 * 128 * 128)
    assert st == sf.SF_ERR_INVALID and "state_pool" in err
    st, err = call(pool=FAKE * 16)
    assert st == sf.SF_ERR_INVALID and "state_indices" in err
    st, err = call(q=None)
    assert st == sf.SF_ERR_INVALID and "NULL" in err


def test_gate_transform_rejects_invalid_arguments(L):
    call = lambda dt=sf.SF_BF16, kind=sf.SF_GATE_BOUNDED, lb=-5.0, raw=FAKE * 16, out=FAKE * 16, H=4, D=1: \
        L.sf_gate_transform(dt, raw, FAKE, FAKE, 8, H, D, kind, lb, out, None)
    assert call(kind=7) == sf.SF_ERR_INVALID
    assert call(lb=1.0) == sf.SF_ERR_INVALID
    assert call(lb=float("-inf")) == sf.SF_ERR_INVALID
    assert call(lb=float("nan")) == sf.SF_ERR_INVALID
    assert call(raw=FAKE * 16 + 4) == sf.SF_ERR_INVALID          # misaligned
    assert call(raw=None) == sf.SF_ERR_INVALID
    assert call(H=0) == sf.SF_ERR_INVALID
    assert L.sf_gate_transform(sf.SF_F32, None, None, None, 0, 4, 1, sf.SF_GATE_SOFTPLUS, 0.0, None, None) == sf.SF_OK
    with pytest.raises(ValueError, match="lower_bound"):
        sf.gate_transform(None, None, None, kind="softplus", lower_bound=-1.0)
    with pytest.raises(ValueError, match="kind"):
        sf.gate_transform(None, None, None, kind="linear")


def test_paged_chunk_rejects_invalid_arguments(L):
    def call(stride=4 * 128 * 128, pool=FAKE * 16, idx=FAKE, K=128, V=128, ws=FAKE * 256, nbytes=1 << 40):
        st = L.sf_paged_gdn_chunk_fwd(sf.SF_BF16, FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 2, 128, 4, 4, K, V, 1.0, FAKE,
                                      pool, sf.SF_F32, 9, stride, idx, None, ws, nbytes, None)
        return st, L.sf_last_error().decode()
    assert call(K=96, V=96)[0] == sf.SF_ERR_UNSUPPORTED
    assert call(stride=100)[0] == sf.SF_ERR_INVALID
    assert call(idx=None)[0] == sf.SF_ERR_INVALID
    assert call(pool=FAKE * 16 + 4)[0] == sf.SF_ERR_INVALID
    assert call(nbytes=16)[0] == sf.SF_ERR_WORKSPACE
    need = L.sf_paged_gdn_chunk_fwd_workspace(sf.SF_BF16, 2, 128, 4, 128, 128, 2, 0)
    assert need == L.sf_gdn_chunk_fwd_workspace(sf.SF_BF16, 2, 128, 4, 128, 128, 2, 0) + 2 * (2 * 4 * 128 * 128 * 4)


def test_raw_gate_chunk_rejects_invalid_arguments(L):
    def call(kind=sf.SF_GATE_SOFTPLUS, lb=0.0, raw=FAKE, K=128):
        return L.sf_gdn_chunk_fwd_raw_gate(sf.SF_BF16, FAKE, FAKE, FAKE, raw, FAKE, FAKE, kind, lb, FAKE, None, None, 2,
                                           2, 128, 4, 4, K, K, 1.0, FAKE, None, FAKE * 256, 1 << 40, None)
    assert call(raw=None) == sf.SF_ERR_INVALID
    assert call(kind=5) == sf.SF_ERR_INVALID
    assert call(kind=sf.SF_GATE_BOUNDED, lb=2.0) == sf.SF_ERR_INVALID
    assert call(K=96) == sf.SF_ERR_UNSUPPORTED


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 64, 2, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        sf.gdn_chunk_fwd(q, q, q, torch.zeros(1, 64, 2), torch.zeros(1, 64, 2))


def test_segment_view_indexing():
    """Row s = b*n_seg + j of the segment view covers tokens [j*L, (j+1)*L) of batch row b."""
    import torch
    B, T, n_seg = 3, 48, 4
    x = torch.arange(B * T * 2).view(B, T, 2)
    sv = sf.segment_view(x, n_seg)
    L = T // n_seg
    for b in range(B):
        for j in range(n_seg):
            assert torch.equal(sv[b * n_seg + j], x[b, j * L:(j + 1) * L])
            assert sv[b * n_seg + j].data_ptr() == x[b, j * L].data_ptr()


def test_host_validators(L):
    """The debug checks on host copies of cu_seqlens and slot indices (no GPU, nothing enqueued)."""
    import numpy as np

    def cu_ok(arr, T):
        a = np.ascontiguousarray(np.asarray(arr, dtype=np.int32))
        return L.sf_check_cu_seqlens(a.ctypes.data_as(ctypes.c_void_p), len(a) - 1, T)

    assert cu_ok([0, 5, 5, 9], 9) == sf.SF_OK
    assert cu_ok([0], 0) == sf.SF_OK
    assert cu_ok([1, 5], 9) == sf.SF_ERR_INVALID and b"cu_seqlens[0]" in L.sf_last_error()
    assert cu_ok([0, 5, 4], 9) == sf.SF_ERR_INVALID and b"decreases" in L.sf_last_error()
    assert cu_ok([0, 5, 10], 9) == sf.SF_ERR_INVALID and b"past T" in L.sf_last_error()

    def idx_ok(arr, ns):
        a = np.ascontiguousarray(np.asarray(arr, dtype=np.int32))
        return L.sf_check_state_indices(a.ctypes.data_as(ctypes.c_void_p), len(a), ns)

    assert idx_ok([3, 0, -1, 1, 2], 4) == sf.SF_OK
    assert idx_ok([3, 4], 4) == sf.SF_ERR_INVALID and b"past num_slots" in L.sf_last_error()
    assert idx_ok([2, 0, 2], 4) == sf.SF_ERR_INVALID and b"race" in L.sf_last_error()
    # the binding's helpers raise on the same cases (host tensors: no GPU needed)
    import torch
    sf.validate_cu_seqlens(torch.tensor([0, 3, 3], dtype=torch.int32), 3)
    with pytest.raises(sf.SfError):
        sf.validate_cu_seqlens(torch.tensor([0, 3, 2], dtype=torch.int32), 3)
    with pytest.raises(sf.SfError):
        sf.validate_state_indices(torch.tensor([1, 1], dtype=torch.int32), 4)


def test_noalloc_rejects_sizes_past_its_scratch(L):
    """sf_gdn_chunk_fwd_noalloc refuses, on the host, sizes whose workspace exceeds its static array."""
    assert L.sf_static_scratch_bytes() == 64 << 20
    st = L.sf_gdn_chunk_fwd_noalloc(sf.SF_BF16, *([ctypes.c_void_p(FAKE)] * 5), None, None, 1, 1, 1 << 18, 16, 16,
                                    128, 128, ctypes.c_float(0.1), ctypes.c_void_p(FAKE), None, None)
    assert st == sf.SF_ERR_WORKSPACE and b"static" in L.sf_last_error()


def test_bwd_workspace_size(L):
    # float32 records (T [64][64], W and Qt [64][K], 256 coefficients), entry states and exit-state gradients
    B, T, H, K, V = 2, 4096, 16, 128, 128
    slots = B * (T // 64)
    rec = 4 * (64 * 64 + 2 * 64 * K + 256)
    al = lambda x: (x + 255) // 256 * 256
    want = al(slots * H * rec) + 2 * al(slots * H * V * K * 4)
    assert L.sf_gdn_chunk_bwd_workspace(sf.SF_BF16, B, T, H, K, V, B, 0) == want
    assert L.sf_gdn_chunk_bwd_workspace(7, B, T, H, K, V, B, 0) == 0


def bwd_call(L, **kw):
    a = dict(dt=sf.SF_BF16, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, dout=FAKE, dht=None, cu=None,
             N=1, B=1, T=128, H=4, HK=4, K=128, V=128, scale=ctypes.c_float(0.1), dq=FAKE, dk=FAKE, dv=FAKE,
             dg=FAKE, dbeta=FAKE, dh0=None, ws=FAKE * 256, wsb=1 << 40, s=None)
    a.update(kw)
    st = L.sf_gdn_chunk_bwd(a["dt"], a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["dout"], a["dht"], a["cu"],
                            a["N"], a["B"], a["T"], a["H"], a["HK"], a["K"], a["V"], a["scale"], a["dq"], a["dk"],
                            a["dv"], a["dg"], a["dbeta"], a["dh0"], a["ws"], a["wsb"], a["s"])
    return st, L.sf_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(HK=2), sf.SF_ERR_UNSUPPORTED, "one q/k head per value head"),
    (dict(HK=3), sf.SF_ERR_INVALID, "divide"),
    (dict(dout=None), sf.SF_ERR_INVALID, "NULL"),
    (dict(dbeta=None), sf.SF_ERR_INVALID, "NULL"),
    (dict(K=96), sf.SF_ERR_UNSUPPORTED, "{64, 128}"),
    (dict(V=32), sf.SF_ERR_UNSUPPORTED, "{64, 128}"),
    (dict(wsb=16), sf.SF_ERR_WORKSPACE, "smaller"),
    (dict(ws=FAKE * 256 + 8), sf.SF_ERR_INVALID, "aligned"),
    (dict(dq=FAKE + 2), sf.SF_ERR_INVALID, "16-byte aligned"),
    (dict(v=FAKE + 8), sf.SF_ERR_INVALID, "16-byte aligned"),
    (dict(N=3), sf.SF_ERR_INVALID, "N (3) must equal B"),
])
def test_bwd_rejects_invalid_arguments(L, kw, status, msg):
    st, err = bwd_call(L, **kw)
    assert st == status, err
    assert msg in err


def test_kda_chunk_workspace_size(L):
    B, T, H, K, V = 2, 4096, 16, 128, 128
    slots = B * (T // 64)
    rec = 4 * (3 * 64 * K + 64 * V + 64 * 64 + K)   # W, Qg, Kh [64][K]; U [64][V]; P [64][64]; Gamma_L [K]
    al = lambda x: (x + 255) // 256 * 256
    assert L.sf_kda_chunk_fwd_workspace(sf.SF_BF16, B, T, H, K, V, B, 0) == al(slots * H * rec)
    assert L.sf_kda_chunk_fwd_workspace(sf.SF_BF16, B, T, H, 64, 128, B, 0) == 0


def kda_call(L, **kw):
    a = dict(dt=sf.SF_BF16, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, cu=None, N=1, B=1, T=128, H=4,
             K=128, V=128, scale=ctypes.c_float(0.1), out=FAKE, ht=None, ws=FAKE * 256, wsb=1 << 40, s=None)
    a.update(kw)
    st = L.sf_kda_chunk_fwd(a["dt"], a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["cu"], a["N"], a["B"],
                            a["T"], a["H"], a["K"], a["V"], a["scale"], a["out"], a["ht"], a["ws"], a["wsb"], a["s"])
    return st, L.sf_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=64, V=128), sf.SF_ERR_UNSUPPORTED, "(K, V)"),
    (dict(K=96, V=96), sf.SF_ERR_UNSUPPORTED, "(K, V)"),
    (dict(g=None), sf.SF_ERR_INVALID, "NULL"),
    (dict(out=None), sf.SF_ERR_INVALID, "NULL"),
    (dict(wsb=16), sf.SF_ERR_WORKSPACE, "smaller"),
    (dict(ws=FAKE * 256 + 8), sf.SF_ERR_INVALID, "aligned"),
    (dict(cu=FAKE, B=2, N=2), sf.SF_ERR_INVALID, "batch-one"),
    (dict(k=FAKE + 4), sf.SF_ERR_INVALID, "16-byte aligned"),
])
def test_kda_chunk_rejects_invalid_arguments(L, kw, status, msg):
    st, err = kda_call(L, **kw)
    assert st == status, err
    assert msg in err

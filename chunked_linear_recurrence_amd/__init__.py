"""Chunk-parallel linear recurrences on MI355X (gfx950): Python binding.

This module only marshals arguments: it checks tensor shapes and dtypes,
allocates outputs and workspaces with PyTorch (which is used here for device
memory and streams only) and calls the C ABI of ``libsf.so`` (include/sf.h)
on the current HIP stream. Every step of the computation runs in the HIP
kernels of that library; there is no CPU or PyTorch fallback, and a missing
library is an error.

Functions (same names as the C entry points, without the ``sf_`` prefix):

* ``gdn_chunk_fwd``     Gated Delta Rule forward, 64-token chunks
                        (attention-gym "Linear Attention", "Gated Delta Rule").
* ``gdn_chunk_bwd``     its gradients (dq, dk, dv, dg, dbeta, dh0), the state
                        gradient carried from the last chunk back to the first
                        (StateFlow Section 2.2, Eq. (6)-(7)).
* ``gla_chunk_fwd``     scalar-gated linear attention forward
                        (StateFlow Eq. (1), scalar-identity transition).
* ``segment_summary``   affine summary per segment row (attention-gym
                        "Context Parallelism"; Megatron-LM "Mamba2 state-passing
                        context parallelism").
* ``state_scan``        exclusive scan over segment summaries.
* ``segmented_gdn_fwd`` / ``segmented_gla_fwd``: one long sequence cut into
  segments laid along the batch axis: summary -> scan -> chunk forward.
* ``gdn_decode``        one-token paged Gated Delta Rule decode (attention-gym
                        "Linear Attention", recurrent_gdn_decode).
* ``gdn_recurrent_fwd`` token-by-token Gated Delta Rule forward, optionally on a
                        paged state pool (attention-gym "Linear Attention",
                        recurrent_gdn).
* ``paged_gdn_chunk_fwd`` chunk forward on a paged state cache (attention-gym
                        "Linear Attention", paged_chunk_gdn).
* ``gdn_chunk_fwd_raw_gate`` gdn_chunk_fwd with the gate transform fused into its
                        Pre stage (raw gate projection in, no separate kernel).
* ``kda_chunk_fwd``     Kimi Delta Attention forward in 64-token chunks
                        (attention-gym "Linear Attention", chunk_kda).
* ``kda_recurrent_fwd`` Kimi Delta Attention token by token (per-channel gate),
                        optionally on a paged state pool.
* ``kda_decode``        one-token paged KDA decode (recurrent_kda_decode).
* ``gate_transform``    raw gate projections to float32 natural-log decays
                        (attention-gym "Linear Attention", "Gate Transforms").
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsf.so")

SF_OK, SF_ERR_INVALID, SF_ERR_UNSUPPORTED, SF_ERR_HIP, SF_ERR_WORKSPACE = range(5)
SF_F32, SF_BF16 = 0, 1
SF_KIND_GDN, SF_KIND_GLA = 0, 1
SF_GATE_SOFTPLUS, SF_GATE_BOUNDED = 0, 1
GATE_KINDS = {"softplus": SF_GATE_SOFTPLUS, "bounded": SF_GATE_BOUNDED}
KINDS = {"gdn": SF_KIND_GDN, "gla": SF_KIND_GLA}

EXPORTED = (
    "sf_version", "sf_last_error", "sf_gdn_chunk_fwd_workspace", "sf_gdn_chunk_fwd",
    "sf_gla_chunk_fwd", "sf_segment_summary_workspace", "sf_segment_summary",
    "sf_state_scan", "sf_gdn_segmented_fwd_workspace", "sf_gdn_segmented_fwd", "sf_gdn_decode", "sf_gdn_recurrent_fwd", "sf_gate_transform",
    "sf_paged_gdn_chunk_fwd_workspace", "sf_paged_gdn_chunk_fwd", "sf_gdn_chunk_fwd_raw_gate",
    "sf_kda_recurrent_fwd", "sf_kda_decode",
    "sf_timing_enable", "sf_timing_collect", "sf_check_cu_seqlens", "sf_check_state_indices",
    "sf_gdn_chunk_fwd_noalloc", "sf_static_scratch_bytes", "sf_gdn_chunk_bwd_workspace", "sf_gdn_chunk_bwd",
    "sf_kda_chunk_fwd_workspace", "sf_kda_chunk_fwd",
)


class SfError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sf status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsf.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m chunked_linear_recurrence_amd.build` "
            "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.sf_version.restype = ctypes.c_char_p
    L.sf_last_error.restype = ctypes.c_char_p
    L.sf_gdn_chunk_fwd_workspace.restype = Z
    L.sf_gdn_chunk_fwd_workspace.argtypes = [I, I, I, I, I, I, I, I]
    L.sf_gdn_chunk_fwd.restype = I
    L.sf_gdn_chunk_fwd.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P, Z, P]
    L.sf_gla_chunk_fwd.restype = I
    L.sf_gla_chunk_fwd.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P, P, P]
    L.sf_segment_summary_workspace.restype = Z
    L.sf_segment_summary_workspace.argtypes = [I, I, I, I, I, I, I, I]
    L.sf_segment_summary.restype = I
    L.sf_segment_summary.argtypes = [I, I, P, P, P, P, I, I, I, I, I, I, I, P, P, P, Z, P]
    L.sf_state_scan.restype = I
    L.sf_state_scan.argtypes = [I, P, P, P, I, I, I, I, I, P, P, P]
    L.sf_gdn_segmented_fwd_workspace.restype = Z
    L.sf_gdn_segmented_fwd_workspace.argtypes = [I, I, I, I, I, I, I]
    L.sf_gdn_segmented_fwd.restype = I
    L.sf_gdn_segmented_fwd.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P, Z, P]
    L.sf_gdn_decode.restype = I
    L.sf_gdn_decode.argtypes = [I, P, P, P, P, P, P, I, I, ctypes.c_longlong, P, P, I, I, I, I, I, F, P, P]
    L.sf_gdn_recurrent_fwd.restype = I
    L.sf_gdn_recurrent_fwd.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P, I, I,
                                       ctypes.c_longlong, P, P, P]
    L.sf_paged_gdn_chunk_fwd_workspace.restype = Z
    L.sf_paged_gdn_chunk_fwd_workspace.argtypes = [I, I, I, I, I, I, I, I]
    L.sf_paged_gdn_chunk_fwd.restype = I
    L.sf_paged_gdn_chunk_fwd.argtypes = [I, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, I, I, ctypes.c_longlong,
                                         P, P, P, Z, P]
    L.sf_gdn_chunk_fwd_raw_gate.restype = I
    L.sf_gdn_chunk_fwd_raw_gate.argtypes = [I, P, P, P, P, P, P, I, F, P, P, P, I, I, I, I, I, I, I, F, P, P, P, Z, P]
    L.sf_kda_recurrent_fwd.restype = I
    L.sf_kda_recurrent_fwd.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, I, I,
                                       ctypes.c_longlong, P, P, P]
    L.sf_kda_decode.restype = I
    L.sf_kda_decode.argtypes = [I, P, P, P, P, P, I, F, P, I, I, ctypes.c_longlong, P, P, I, I, I, I, F, P, P]
    L.sf_gate_transform.restype = I
    L.sf_gate_transform.argtypes = [I, P, P, P, ctypes.c_longlong, I, I, I, F, P, P]
    L.sf_gdn_chunk_fwd_noalloc.restype = I
    L.sf_gdn_chunk_fwd_noalloc.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P]
    L.sf_static_scratch_bytes.restype = Z
    L.sf_static_scratch_bytes.argtypes = []
    L.sf_kda_chunk_fwd_workspace.restype = Z
    L.sf_kda_chunk_fwd_workspace.argtypes = [I, I, I, I, I, I, I, I]
    L.sf_kda_chunk_fwd.restype = I
    L.sf_kda_chunk_fwd.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, P, P, Z, P]
    L.sf_gdn_chunk_bwd_workspace.restype = Z
    L.sf_gdn_chunk_bwd_workspace.argtypes = [I, I, I, I, I, I, I, I]
    L.sf_gdn_chunk_bwd.restype = I
    L.sf_gdn_chunk_bwd.argtypes = [I, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, P, P, P, P, P, P, Z, P]
    L.sf_check_cu_seqlens.restype = I
    L.sf_check_cu_seqlens.argtypes = [P, I, I]
    L.sf_check_state_indices.restype = I
    L.sf_check_state_indices.argtypes = [P, I, I]
    L.sf_timing_enable.restype = I
    L.sf_timing_enable.argtypes = [I]
    L.sf_timing_collect.restype = I
    L.sf_timing_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int), I]
    _lib = L
    return L


def version() -> str:
    return lib().sf_version().decode()


def _check(status: int):
    if status != SF_OK:
        raise SfError(status, lib().sf_last_error().decode())


def validate_cu_seqlens(cu_seqlens: torch.Tensor, T: int) -> None:
    """Debug check of packed offsets (copies them to the host, which synchronises): starts at 0, never
    decreases, ends at or before T. Raises SfError otherwise."""
    h = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    _check(lib().sf_check_cu_seqlens(ctypes.c_void_p(h.data_ptr()), h.numel() - 1, int(T)))


def validate_state_indices(state_indices: torch.Tensor, num_slots: int) -> None:
    """Debug check of slot indices (copies them to the host): positive indices below num_slots and
    unique. Raises SfError otherwise."""
    h = state_indices.detach().to("cpu", torch.int32).contiguous()
    _check(lib().sf_check_state_indices(ctypes.c_void_p(h.data_ptr()), h.numel(), int(num_slots)))


def _validating() -> bool:
    return os.environ.get("SF_VALIDATE", "0") == "1"


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SF_BF16
    if t.dtype == torch.float32:
        return SF_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _need(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _token_args(q, k, v, g, beta, initial_state, cu_seqlens, g_dtype=torch.float32):
    _need(q, "q", ndim=4)
    dev = q.device
    _need(k, "k", dtype=q.dtype, ndim=4, device=dev)
    _need(v, "v", dtype=q.dtype, ndim=4, device=dev)
    _need(g, "g", dtype=g_dtype, ndim=3, device=dev)
    if beta is not None:
        _need(beta, "beta", dtype=torch.float32, ndim=3, device=dev)
    B, T, HK, K = q.shape
    H, V = v.shape[2], v.shape[3]
    if k.shape != q.shape or v.shape[:2] != (B, T) or g.shape != (B, T, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)} g {tuple(g.shape)}")
    if beta is not None and beta.shape != g.shape:
        raise ValueError("beta must have the shape of g")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1, device=dev)
        N = cu_seqlens.numel() - 1
        if _validating():
            validate_cu_seqlens(cu_seqlens, T)
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", dtype=torch.float32, ndim=4, device=dev)
        if tuple(initial_state.shape) != (N, H, V, K):
            raise ValueError(f"initial_state must be [{N}, {H}, {V}, {K}], got {tuple(initial_state.shape)}")
    return B, T, H, HK, K, V, N


def gdn_chunk_fwd(q, k, v, g, beta, initial_state=None, *, cu_seqlens=None, scale=None,
                  output_final_state=False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Gated Delta Rule chunk forward. q, k [B,T,HK,K]; v [B,T,H,V]; g, beta [B,T,H] float32;
    initial_state [N,H,V,K] float32. Returns (output [B,T,H,V] in q.dtype, final state or None).
    Output rows at or past cu_seqlens[-1] are left uninitialised."""
    B, T, H, HK, K, V, N = _token_args(q, k, v, g, beta, initial_state, cu_seqlens)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    dev = q.device
    out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
    ht = torch.empty((N, H, V, K), dtype=torch.float32, device=dev) if output_final_state else None
    dt = _dt(q)
    nbytes = lib().sf_gdn_chunk_fwd_workspace(dt, B, T, H, K, V, N, int(cu_seqlens is not None))
    ws = _workspace(nbytes, dev)
    _check(lib().sf_gdn_chunk_fwd(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                  _ptr(cu_seqlens), N, B, T, H, HK, K, V, float(scale), _ptr(out), _ptr(ht),
                                  _ptr(ws), nbytes, _stream()))
    return out, ht


def gdn_chunk_bwd(q, k, v, g, beta, do, initial_state=None, dht=None, *, cu_seqlens=None, scale=None):
    """Gated Delta Rule chunk backward: the gradients of sum(do * o) + sum(dht * ht) for the forward of
    gdn_chunk_fwd with the same arguments. do [B,T,H,V] in q.dtype; dht [N,H,V,K] float32 or None.
    Returns (dq, dk, dv in q.dtype, dg, dbeta float32 [B,T,H], dh0 float32 [N,H,V,K]). Entries of tokens at
    or past cu_seqlens[-1] are left uninitialised. Needs HK == H."""
    B, T, H, HK, K, V, N = _token_args(q, k, v, g, beta, initial_state, cu_seqlens)
    dev = q.device
    _need(do, "do", dtype=q.dtype, ndim=4, device=dev)
    if tuple(do.shape) != (B, T, H, V):
        raise ValueError(f"do must be [{B}, {T}, {H}, {V}], got {tuple(do.shape)}")
    if dht is not None:
        _need(dht, "dht", dtype=torch.float32, ndim=4, device=dev)
        if tuple(dht.shape) != (N, H, V, K):
            raise ValueError(f"dht must be [{N}, {H}, {V}, {K}], got {tuple(dht.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dbeta = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dh0 = torch.empty((N, H, V, K), dtype=torch.float32, device=dev)
    dt = _dt(q)
    nbytes = lib().sf_gdn_chunk_bwd_workspace(dt, B, T, H, K, V, N, int(cu_seqlens is not None))
    ws = _workspace(nbytes, dev)
    _check(lib().sf_gdn_chunk_bwd(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(do),
                                  _ptr(dht), _ptr(cu_seqlens), N, B, T, H, HK, K, V, float(scale), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(ws), nbytes, _stream()))
    return dq, dk, dv, dg, dbeta, dh0


def kda_chunk_fwd(q, k, v, g, beta, initial_state=None, *, cu_seqlens=None, scale=None, output_final_state=False):
    """Kimi Delta Attention chunk forward: q, k, g [B,T,H,K] (g float32, per-channel natural-log decay),
    v [B,T,H,V], beta [B,T,H] float32, initial_state [N,H,V,K] float32. Returns (output [B,T,H,V] in q.dtype,
    final state or None). Output rows at or past cu_seqlens[-1] are left uninitialised."""
    _need(q, "q", ndim=4)
    dev = q.device
    _need(k, "k", dtype=q.dtype, ndim=4, device=dev)
    _need(v, "v", dtype=q.dtype, ndim=4, device=dev)
    _need(g, "g", dtype=torch.float32, ndim=4, device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=3, device=dev)
    B, T, H, K = q.shape
    V = v.shape[3]
    if k.shape != q.shape or g.shape != q.shape or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} g {tuple(g.shape)} v {tuple(v.shape)} "
                         f"beta {tuple(beta.shape)}")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1, device=dev)
        N = cu_seqlens.numel() - 1
        if _validating():
            validate_cu_seqlens(cu_seqlens, T)
    else:
        N = B
    if initial_state is not None:
        _need(initial_state, "initial_state", dtype=torch.float32, ndim=4, device=dev)
        if tuple(initial_state.shape) != (N, H, V, K):
            raise ValueError(f"initial_state must be [{N}, {H}, {V}, {K}], got {tuple(initial_state.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
    ht = torch.empty((N, H, V, K), dtype=torch.float32, device=dev) if output_final_state else None
    dt = _dt(q)
    nbytes = lib().sf_kda_chunk_fwd_workspace(dt, B, T, H, K, V, N, int(cu_seqlens is not None))
    ws = _workspace(nbytes, dev)
    _check(lib().sf_kda_chunk_fwd(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                  _ptr(cu_seqlens), N, B, T, H, K, V, float(scale), _ptr(out), _ptr(ht), _ptr(ws),
                                  nbytes, _stream()))
    return out, ht


def gdn_chunk_fwd_raw_gate(q, k, v, raw_gate, A_log, dt_bias, beta, initial_state=None, *, kind,
                           lower_bound=None, cu_seqlens=None, scale=None, output_final_state=False):
    """gdn_chunk_fwd whose natural-log gate is formed inside the kernels from raw_gate [B,T,H] (q's dtype),
    A_log [H] and dt_bias [H] (float32): kind "softplus" or "bounded" (with lower_bound), as gate_transform."""
    if kind not in GATE_KINDS:
        raise ValueError(f"kind must be one of {sorted(GATE_KINDS)}, got {kind!r}")
    if kind == "softplus" and lower_bound is not None:
        raise ValueError("lower_bound is rejected by the softplus kind")
    if kind == "bounded" and (lower_bound is None or not math.isfinite(lower_bound) or lower_bound > 0):
        raise ValueError("the bounded kind needs a finite lower_bound <= 0")
    B, T, H, HK, K, V, N = _token_args(q, k, v, raw_gate, beta, initial_state, cu_seqlens, g_dtype=q.dtype)
    _need(A_log, "A_log", dtype=torch.float32, ndim=1, device=q.device)
    _need(dt_bias, "dt_bias", dtype=torch.float32, ndim=1, device=q.device)
    if A_log.numel() != H or dt_bias.numel() != H:
        raise ValueError(f"A_log and dt_bias must have {H} entries")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    dev = q.device
    out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
    ht = torch.empty((N, H, V, K), dtype=torch.float32, device=dev) if output_final_state else None
    dt = _dt(q)
    nbytes = lib().sf_gdn_chunk_fwd_workspace(dt, B, T, H, K, V, N, int(cu_seqlens is not None))
    ws = _workspace(nbytes, dev)
    _check(lib().sf_gdn_chunk_fwd_raw_gate(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(A_log), _ptr(dt_bias),
                                           GATE_KINDS[kind], float(lower_bound or 0.0), _ptr(beta), _ptr(initial_state),
                                           _ptr(cu_seqlens), N, B, T, H, HK, K, V, float(scale), _ptr(out), _ptr(ht),
                                           _ptr(ws), nbytes, _stream()))
    return out, ht


def gla_chunk_fwd(q, k, v, g, initial_state=None, *, cu_seqlens=None, scale=1.0, chunk=64,
                  output_final_state=False):
    """Scalar-gated linear attention forward: S_t = exp(g_t) S_{t-1} + v_t k_t^T,
    o_t = scale S_t q_t. Returns (output, final state or None)."""
    B, T, H, HK, K, V, N = _token_args(q, k, v, g, None, initial_state, cu_seqlens)
    dev = q.device
    out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
    ht = torch.empty((N, H, V, K), dtype=torch.float32, device=dev) if output_final_state else None
    _check(lib().sf_gla_chunk_fwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(initial_state),
                                  _ptr(cu_seqlens), N, B, T, H, HK, K, V, int(chunk), float(scale), _ptr(out),
                                  _ptr(ht), _stream()))
    return out, ht


def segment_summary(kind, k, v, g, beta=None, *, chunk=None):
    """Affine summary of each row of [n_rows, L_seg, ...] inputs.
    kind "gdn": returns (M [n_rows,H,K,K], S_ext [n_rows,H,V,K]);
    kind "gla": returns (a_block [n_rows,H], S_ext)."""
    kd = KINDS[kind]
    _need(k, "k", ndim=4)
    dev = k.device
    _need(v, "v", dtype=k.dtype, ndim=4, device=dev)
    _need(g, "g", dtype=torch.float32, ndim=3, device=dev)
    R, L, HK, K = k.shape
    H, V = v.shape[2], v.shape[3]
    if v.shape[:2] != (R, L) or g.shape != (R, L, H):
        raise ValueError("shape mismatch between k, v and g")
    if kd == SF_KIND_GDN:
        _need(beta, "beta", dtype=torch.float32, ndim=3, device=dev)
        if beta.shape != g.shape:
            raise ValueError("beta must have the shape of g")
    chunk = chunk or 64
    dt = _dt(k)
    M = torch.empty((R, H, K, K) if kd == SF_KIND_GDN else (R, H), dtype=torch.float32, device=dev)
    S_ext = torch.empty((R, H, V, K), dtype=torch.float32, device=dev)
    nbytes = lib().sf_segment_summary_workspace(kd, dt, R, L, H, K, V, chunk)
    ws = _workspace(nbytes, dev) if nbytes else None
    _check(lib().sf_segment_summary(kd, dt, _ptr(k), _ptr(v), _ptr(g), _ptr(beta), R, L, H, HK, K, V, chunk,
                                    _ptr(M), _ptr(S_ext), _ptr(ws), nbytes, _stream()))
    return M, S_ext


def state_scan(kind, M, S_ext, h0=None, *, B, n_seg, final_state=True):
    """Exclusive scan over segment rows s = b*n_seg + j. Returns (S_in, S_final or None)."""
    kd = KINDS[kind]
    _need(S_ext, "S_ext", dtype=torch.float32, ndim=4)
    dev = S_ext.device
    _need(M, "M", dtype=torch.float32, device=dev)
    R, H, V, K = S_ext.shape
    if R != B * n_seg:
        raise ValueError(f"S_ext has {R} rows, expected B*n_seg = {B * n_seg}")
    want_M = (R, H, K, K) if kd == SF_KIND_GDN else (R, H)
    if tuple(M.shape) != want_M:
        raise ValueError(f"M must be {want_M}, got {tuple(M.shape)}")
    if h0 is not None:
        _need(h0, "h0", dtype=torch.float32, ndim=4, device=dev)
        if tuple(h0.shape) != (B, H, V, K):
            raise ValueError("h0 must be [B, H, V, K]")
    S_in = torch.empty_like(S_ext)
    S_final = torch.empty((B, H, V, K), dtype=torch.float32, device=dev) if final_state else None
    _check(lib().sf_state_scan(kd, _ptr(M), _ptr(S_ext), _ptr(h0), B, n_seg, H, K, V, _ptr(S_in), _ptr(S_final),
                               _stream()))
    return S_in, S_final


def segment_view(x: torch.Tensor, n_seg: int) -> torch.Tensor:
    """[B, T, ...] -> [B*n_seg, T/n_seg, ...] (a view; row s = b*n_seg + j)."""
    B, T = x.shape[:2]
    if T % n_seg:
        raise ValueError(f"T={T} is not a multiple of n_seg={n_seg}")
    return x.view(B * n_seg, T // n_seg, *x.shape[2:])


def segmented_gdn_fwd(q, k, v, g, beta, n_seg, initial_state=None, *, scale=None, output_final_state=False):
    """One long Gated Delta Rule run cut into n_seg segments per batch row (summary -> scan -> forward,
    one sf_gdn_segmented_fwd call). Equals gdn_chunk_fwd on the whole rows up to floating-point order."""
    B, T, H, HK, K, V, N = _token_args(q, k, v, g, beta, initial_state, None)
    if n_seg <= 0 or T % n_seg or (T // n_seg) % 64:
        raise ValueError("T must split into n_seg segments whose length is a multiple of the 64-token chunk")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    dev = q.device
    out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
    ht = torch.empty((B, H, V, K), dtype=torch.float32, device=dev) if output_final_state else None
    dt = _dt(q)
    nbytes = lib().sf_gdn_segmented_fwd_workspace(dt, B, n_seg, T, H, K, V)
    ws = _workspace(nbytes, dev)
    _check(lib().sf_gdn_segmented_fwd(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), B,
                                      n_seg, T, H, HK, K, V, float(scale), _ptr(out), _ptr(ht), _ptr(ws), nbytes,
                                      _stream()))
    return out, ht


def segmented_gla_fwd(q, k, v, g, n_seg, initial_state=None, *, scale=1.0, chunk=64, output_final_state=False):
    """Scalar-gate counterpart of segmented_gdn_fwd (a_block summaries)."""
    B, T = q.shape[:2]
    if (T // n_seg) % chunk:
        raise ValueError("segment length must be a multiple of the chunk")
    sv = lambda x: segment_view(x, n_seg)
    a, S_ext = segment_summary("gla", sv(k), sv(v), sv(g), chunk=chunk)
    S_in, S_final = state_scan("gla", a, S_ext, initial_state, B=B, n_seg=n_seg, final_state=output_final_state)
    o, _ = gla_chunk_fwd(sv(q), sv(k), sv(v), sv(g), S_in, scale=scale, chunk=chunk)
    return o.view(B, T, *o.shape[2:]), S_final


def _pool_layout(pool, H, V, K, dev):
    if not isinstance(pool, torch.Tensor) or not pool.is_cuda or pool.dim() != 4:
        raise ValueError("the state pool must be a [num_slots, H, V, K] GPU tensor")
    if pool.device != dev:
        raise ValueError(f"the state pool is on {pool.device}, expected {dev}")
    if pool.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"the state pool must be float32 or bfloat16, got {pool.dtype}")
    NS = pool.shape[0]
    if tuple(pool.shape[1:]) != (H, V, K):
        raise ValueError(f"the state pool must be [num_slots, {H}, {V}, {K}], got {tuple(pool.shape)}")
    st = pool.stride()
    if st[3] != 1 or st[2] != K or st[1] != V * K or (NS > 1 and st[0] < H * V * K):
        raise ValueError("each [H, V, K] slot of the state pool must be dense")
    pool_dt = SF_BF16 if pool.dtype == torch.bfloat16 else SF_F32
    return NS, (st[0] if NS > 1 else H * V * K), pool_dt


def gdn_recurrent_fwd(q, k, v, g, beta, initial_state=None, *, cu_seqlens=None, scale=None,
                      output_final_state=False, state_indices=None, has_initial_state=None):
    """Token-by-token Gated Delta Rule forward. q, k [B,T,HK,K]; v [B,T,H,V]; g, beta [B,T,H] float32.
    Without state_indices: initial_state [N,H,V,K] float32 or None; returns (output, final state or None).
    With state_indices [N] int32: initial_state is a [num_slots,H,V,K] float32 or bf16 pool advanced in
    place (each sequence's final state overwrites its slot; indices <= 0 give zero output and leave the
    pool alone); has_initial_state [N] bool marks slots to load; output_final_state must be False."""
    if state_indices is None:
        B, T, H, HK, K, V, N = _token_args(q, k, v, g, beta, initial_state, cu_seqlens)
        if has_initial_state is not None:
            raise ValueError("has_initial_state needs state_indices")
    else:
        B, T, H, HK, K, V, N = _token_args(q, k, v, g, beta, None, cu_seqlens)
        if output_final_state:
            raise ValueError("output_final_state is rejected with state_indices: the pool is advanced in place")
        _need(state_indices, "state_indices", dtype=torch.int32, ndim=1, device=q.device)
        if state_indices.numel() != N:
            raise ValueError(f"state_indices must have {N} entries")
        if has_initial_state is not None:
            _need(has_initial_state, "has_initial_state", dtype=torch.bool, ndim=1, device=q.device)
            if has_initial_state.numel() != N:
                raise ValueError(f"has_initial_state must have {N} entries")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    dev = q.device
    out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
    if state_indices is None:
        ht = torch.empty((N, H, V, K), dtype=torch.float32, device=dev) if output_final_state else None
        _check(lib().sf_gdn_recurrent_fwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                          _ptr(cu_seqlens), N, B, T, H, HK, K, V, float(scale), _ptr(out), _ptr(ht),
                                          None, SF_F32, 0, 0, None, None, _stream()))
        return out, ht
    NS, stride0, pool_dt = _pool_layout(initial_state, H, V, K, dev)
    if _validating():
        validate_state_indices(state_indices, NS)
    _check(lib().sf_gdn_recurrent_fwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), None,
                                      _ptr(cu_seqlens), N, B, T, H, HK, K, V, float(scale), _ptr(out), None,
                                      _ptr(initial_state), pool_dt, NS, stride0, _ptr(state_indices),
                                      _ptr(has_initial_state), _stream()))
    return out, None


def paged_gdn_chunk_fwd(q, k, v, g, beta, state_cache, state_indices, *, cu_seqlens=None, has_initial_state=None,
                        scale=None):
    """Delta-rule chunk forward advancing a paged state cache in place (inference prefill). state_cache
    [num_slots, H, V, K] float32 or bf16; state_indices [N] int32 (<= 0: zero output, cache untouched);
    has_initial_state [N] bool or None. Returns the output [B, T, H, V] in q.dtype."""
    B, T, H, HK, K, V, N = _token_args(q, k, v, g, beta, None, cu_seqlens)
    dev = q.device
    _need(state_indices, "state_indices", dtype=torch.int32, ndim=1, device=dev)
    if state_indices.numel() != N:
        raise ValueError(f"state_indices must have {N} entries")
    if has_initial_state is not None:
        _need(has_initial_state, "has_initial_state", dtype=torch.bool, ndim=1, device=dev)
        if has_initial_state.numel() != N:
            raise ValueError(f"has_initial_state must have {N} entries")
    NS, stride0, pool_dt = _pool_layout(state_cache, H, V, K, dev)
    if _validating():
        validate_state_indices(state_indices, NS)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
    dt = _dt(q)
    nbytes = lib().sf_paged_gdn_chunk_fwd_workspace(dt, B, T, H, K, V, N, int(cu_seqlens is not None))
    ws = _workspace(nbytes, dev)
    _check(lib().sf_paged_gdn_chunk_fwd(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, B, T,
                                        H, HK, K, V, float(scale), _ptr(out), _ptr(state_cache), pool_dt, NS, stride0,
                                        _ptr(state_indices), _ptr(has_initial_state), _ptr(ws), nbytes, _stream()))
    return out


def kda_recurrent_fwd(q, k, v, g, beta, initial_state=None, *, cu_seqlens=None, scale=None,
                      output_final_state=False, state_indices=None, has_initial_state=None):
    """Kimi Delta Attention token by token. q, k, g [B,T,H,K] (g float32, one decay per key channel);
    v [B,T,H,V]; beta [B,T,H] float32. State modes as gdn_recurrent_fwd (initial_state [N,H,V,K] float32,
    or a paged pool with state_indices). Returns (output, final state or None)."""
    _need(q, "q", ndim=4)
    dev = q.device
    _need(g, "g", dtype=torch.float32, ndim=4, device=dev)
    if g.shape != q.shape:
        raise ValueError(f"the per-channel gate must be shaped like q {tuple(q.shape)}, got {tuple(g.shape)}")
    B, T, H, K = q.shape
    if k.shape != q.shape or v.dim() != 4 or v.shape[:3] != (B, T, H):
        raise ValueError("q, k [B,T,H,K] and v [B,T,H,V] must share B, T and H (no grouped heads)")
    V = v.shape[3]
    _need(k, "k", dtype=q.dtype, device=dev)
    _need(v, "v", dtype=q.dtype, device=dev)
    _need(beta, "beta", dtype=torch.float32, ndim=3, device=dev)
    if beta.shape != (B, T, H):
        raise ValueError("beta must be [B, T, H]")
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dtype=torch.int32, ndim=1, device=dev)
        N = cu_seqlens.numel() - 1
        if _validating():
            validate_cu_seqlens(cu_seqlens, T)
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    out = torch.empty((B, T, H, V), dtype=q.dtype, device=dev)
    if state_indices is None:
        if has_initial_state is not None:
            raise ValueError("has_initial_state needs state_indices")
        if initial_state is not None:
            _need(initial_state, "initial_state", dtype=torch.float32, ndim=4, device=dev)
            if tuple(initial_state.shape) != (N, H, V, K):
                raise ValueError(f"initial_state must be [{N}, {H}, {V}, {K}]")
        ht = torch.empty((N, H, V, K), dtype=torch.float32, device=dev) if output_final_state else None
        _check(lib().sf_kda_recurrent_fwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                          _ptr(cu_seqlens), N, B, T, H, K, V, float(scale), _ptr(out), _ptr(ht), None,
                                          SF_F32, 0, 0, None, None, _stream()))
        return out, ht
    if output_final_state:
        raise ValueError("output_final_state is rejected with state_indices: the pool is advanced in place")
    _need(state_indices, "state_indices", dtype=torch.int32, ndim=1, device=dev)
    if state_indices.numel() != N:
        raise ValueError(f"state_indices must have {N} entries")
    if has_initial_state is not None:
        _need(has_initial_state, "has_initial_state", dtype=torch.bool, ndim=1, device=dev)
    NS, stride0, pool_dt = _pool_layout(initial_state, H, V, K, dev)
    if _validating():
        validate_state_indices(state_indices, NS)
    _check(lib().sf_kda_recurrent_fwd(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), None, _ptr(cu_seqlens), N,
                                      B, T, H, K, V, float(scale), _ptr(out), None, _ptr(initial_state), pool_dt, NS,
                                      stride0, _ptr(state_indices), _ptr(has_initial_state), _stream()))
    return out, None


def gdn_decode(packed_qkv, raw_gate, raw_beta, A_log, dt_bias, state_cache, state_indices, *,
               has_initial_state=None, scale=None, out=None):
    """One decode token per sequence; advances ``state_cache`` in place.

    packed_qkv [B, 2*HK*K + H*V] (bf16 or float32): per row the query heads, key heads, value heads;
    raw_gate, raw_beta [1, B, H] or [B, H] in packed_qkv's dtype; A_log, dt_bias [H] float32;
    state_cache [num_slots, H, V, K] float32 or bf16 (each slot dense; padding between slots allowed);
    state_indices [B] int32 (<= 0: null row, zero output, cache untouched); has_initial_state [B]
    bool or None. Returns out [1, B, H, V] in packed_qkv's dtype (``out`` itself when given)."""
    _need(packed_qkv, "packed_qkv", ndim=2)
    dev = packed_qkv.device
    B, W = packed_qkv.shape
    if not isinstance(state_cache, torch.Tensor) or not state_cache.is_cuda or state_cache.dim() != 4:
        raise ValueError("state_cache must be a [num_slots, H, V, K] GPU tensor")
    if state_cache.device != dev:
        raise ValueError(f"state_cache is on {state_cache.device}, expected {dev}")
    if state_cache.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"state_cache must be float32 or bfloat16, got {state_cache.dtype}")
    NS, H, V, K = state_cache.shape
    st = state_cache.stride()
    if st[3] != 1 or st[2] != K or st[1] != V * K or (NS > 1 and st[0] < H * V * K):
        raise ValueError("each [H, V, K] slot of state_cache must be dense")
    if (W - H * V) <= 0 or (W - H * V) % (2 * K):
        raise ValueError(f"packed_qkv width {W} does not match 2*HK*{K} + {H}*{V}")
    HK = (W - H * V) // (2 * K)
    for name, t in (("raw_gate", raw_gate), ("raw_beta", raw_beta)):
        _need(t, name, dtype=packed_qkv.dtype, device=dev)
        if t.numel() != B * H:
            raise ValueError(f"{name} must hold [1, {B}, {H}] values, got shape {tuple(t.shape)}")
    _need(A_log, "A_log", dtype=torch.float32, ndim=1, device=dev)
    _need(dt_bias, "dt_bias", dtype=torch.float32, ndim=1, device=dev)
    if A_log.numel() != H or dt_bias.numel() != H:
        raise ValueError(f"A_log and dt_bias must have {H} entries")
    _need(state_indices, "state_indices", dtype=torch.int32, ndim=1, device=dev)
    if state_indices.numel() != B:
        raise ValueError(f"state_indices must have {B} entries")
    if has_initial_state is not None:
        _need(has_initial_state, "has_initial_state", dtype=torch.bool, ndim=1, device=dev)
        if has_initial_state.numel() != B:
            raise ValueError(f"has_initial_state must have {B} entries")
    if _validating():
        validate_state_indices(state_indices, NS)
    if out is None:
        out = torch.empty((1, B, H, V), dtype=packed_qkv.dtype, device=dev)
    else:
        _need(out, "out", dtype=packed_qkv.dtype, device=dev)
        if out.numel() != B * H * V:
            raise ValueError(f"out must hold [1, {B}, {H}, {V}] values")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    pool_dt = SF_BF16 if state_cache.dtype == torch.bfloat16 else SF_F32
    stride0 = st[0] if NS > 1 else H * V * K
    _check(lib().sf_gdn_decode(_dt(packed_qkv), _ptr(packed_qkv), _ptr(raw_gate), _ptr(raw_beta), _ptr(A_log),
                               _ptr(dt_bias), _ptr(state_cache), pool_dt, NS, stride0, _ptr(state_indices),
                               _ptr(has_initial_state), B, H, HK, K, V, float(scale), _ptr(out), _stream()))
    return out


def gate_transform(raw_gate, A_log, dt_bias, *, kind, lower_bound=None):
    """Raw gate projections to float32 natural-log decays. raw_gate [..., H] with dt_bias [H]
    (per-head) or [..., H, D] with dt_bias [H, D] (per-channel), bf16 or float32; A_log [H] float32.
    kind "softplus": -exp(A_log) softplus(raw + dt_bias); "bounded": lower_bound sigmoid(exp(A_log)
    (raw + dt_bias)), with a finite lower_bound <= 0 (required by "bounded", rejected by "softplus")."""
    if kind not in GATE_KINDS:
        raise ValueError(f"kind must be one of {sorted(GATE_KINDS)}, got {kind!r}")
    if kind == "softplus" and lower_bound is not None:
        raise ValueError("lower_bound is rejected by the softplus kind")
    if kind == "bounded" and (lower_bound is None or not math.isfinite(lower_bound) or lower_bound > 0):
        raise ValueError("the bounded kind needs a finite lower_bound <= 0")
    _need(raw_gate, "raw_gate")
    dev = raw_gate.device
    _need(A_log, "A_log", dtype=torch.float32, ndim=1, device=dev)
    _need(dt_bias, "dt_bias", dtype=torch.float32, device=dev)
    H = A_log.numel()
    if dt_bias.dim() == 1:
        D = 1
        if raw_gate.shape[-1] != H or dt_bias.numel() != H:
            raise ValueError(f"per-head gates: raw_gate [..., {H}] and dt_bias [{H}]")
    elif dt_bias.dim() == 2:
        D = dt_bias.shape[1]
        if raw_gate.dim() < 2 or tuple(raw_gate.shape[-2:]) != (H, D) or dt_bias.shape[0] != H:
            raise ValueError(f"per-channel gates: raw_gate [..., {H}, {D}] and dt_bias [{H}, {D}]")
    else:
        raise ValueError("dt_bias must be [H] or [H, D]")
    rows = raw_gate.numel() // (H * D)
    out = torch.empty(raw_gate.shape, dtype=torch.float32, device=dev)
    _check(lib().sf_gate_transform(_dt(raw_gate), _ptr(raw_gate), _ptr(A_log), _ptr(dt_bias), rows, H, D,
                                   GATE_KINDS[kind], float(lower_bound or 0.0), _ptr(out), _stream()))
    return out


def kda_decode(packed_qkv, raw_gate, raw_beta, A_log, dt_bias, state_cache, state_indices, *,
               has_initial_state=None, gate_transform="bounded", lower_bound=-5.0, scale=None, out=None):
    """One KDA decode token per sequence; advances state_cache in place. packed_qkv [B, H*(2K + V)];
    raw_gate [1, B, H, K] or [B, H, K]; raw_beta [1, B, H]; A_log [H]; dt_bias [H, K] (float32);
    gate_transform "bounded" (lower_bound) or "softplus". Returns out [1, B, H, V]."""
    if gate_transform not in GATE_KINDS:
        raise ValueError(f"gate_transform must be one of {sorted(GATE_KINDS)}")
    if gate_transform == "bounded" and (lower_bound is None or not math.isfinite(lower_bound) or lower_bound > 0):
        raise ValueError("the bounded kind needs a finite lower_bound <= 0")
    _need(packed_qkv, "packed_qkv", ndim=2)
    dev = packed_qkv.device
    B, W = packed_qkv.shape
    if not isinstance(state_cache, torch.Tensor) or state_cache.dim() != 4:
        raise ValueError("state_cache must be a [num_slots, H, V, K] GPU tensor")
    NS, H, V, K = state_cache.shape
    NS, stride0, pool_dt = _pool_layout(state_cache, H, V, K, dev)
    if _validating():
        validate_state_indices(state_indices, NS)
    if W != H * (2 * K + V):
        raise ValueError(f"packed_qkv width {W} must be H*(2K + V) = {H * (2 * K + V)}")
    _need(raw_gate, "raw_gate", dtype=packed_qkv.dtype, device=dev)
    if raw_gate.numel() != B * H * K:
        raise ValueError(f"raw_gate must hold [1, {B}, {H}, {K}] values")
    _need(raw_beta, "raw_beta", dtype=packed_qkv.dtype, device=dev)
    if raw_beta.numel() != B * H:
        raise ValueError(f"raw_beta must hold [1, {B}, {H}] values")
    _need(A_log, "A_log", dtype=torch.float32, ndim=1, device=dev)
    _need(dt_bias, "dt_bias", dtype=torch.float32, ndim=2, device=dev)
    if A_log.numel() != H or tuple(dt_bias.shape) != (H, K):
        raise ValueError(f"A_log must be [{H}] and dt_bias [{H}, {K}]")
    _need(state_indices, "state_indices", dtype=torch.int32, ndim=1, device=dev)
    if state_indices.numel() != B:
        raise ValueError(f"state_indices must have {B} entries")
    if has_initial_state is not None:
        _need(has_initial_state, "has_initial_state", dtype=torch.bool, ndim=1, device=dev)
    if out is None:
        out = torch.empty((1, B, H, V), dtype=packed_qkv.dtype, device=dev)
    else:
        _need(out, "out", dtype=packed_qkv.dtype, device=dev)
        if out.numel() != B * H * V:
            raise ValueError(f"out must hold [1, {B}, {H}, {V}] values")
    if scale is None:
        scale = 1.0 / math.sqrt(K)
    _check(lib().sf_kda_decode(_dt(packed_qkv), _ptr(packed_qkv), _ptr(raw_gate), _ptr(raw_beta), _ptr(A_log),
                               _ptr(dt_bias), GATE_KINDS[gate_transform], float(lower_bound or 0.0), _ptr(state_cache),
                               pool_dt, NS, stride0, _ptr(state_indices), _ptr(has_initial_state), B, H, K, V,
                               float(scale), _ptr(out), _stream()))
    return out


def timing_enable(max_pairs: int = 4096):
    """Bracket every library launch with HIP events (0 disables)."""
    _check(lib().sf_timing_enable(int(max_pairs)))


def timing_collect(max_kernels: int = 32):
    """{kernel name: (launches, total ms)} since the last collect (synchronises on the events)."""
    names = (ctypes.c_char_p * max_kernels)()
    ms = (ctypes.c_double * max_kernels)()
    cnt = (ctypes.c_int * max_kernels)()
    n = lib().sf_timing_collect(names, ms, cnt, max_kernels)
    if n < 0:
        raise SfError(SF_ERR_HIP, "timing collect failed")
    return {names[i].decode(): (cnt[i], ms[i]) for i in range(n)}

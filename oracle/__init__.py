"""Oracle for the chunked linear recurrence forward pass (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls it, and it never imports
the product path. It is a plain float64 CPU implementation, written in C in
``oracle.c`` and called here through ctypes on numpy arrays.

What each function follows (pages by title and section):

* ``gdn_forward``   attention-gym "Linear Attention", section "Gated Delta
  Rule": the per-token rule, [N, H, V, K] states, grouped q/k heads,
  cu_seqlens packing.
* ``gla_forward``   StateFlow Section 2.1 Eq. (1) with a scalar-identity
  transition (Mamba-2), the form the Megatron-LM "Mamba2 state-passing
  context parallelism" page summarises.
* ``gdn_summary``   attention-gym "Linear Attention", section "Context
  Parallelism" (affine range map; probe from a zero and an identity entry).
* ``gla_summary``   Megatron-LM "Mamba2 state-passing context parallelism"
  (a_block and S_ext).
* ``state_scan``    the exclusive causal scan of the same page.
* ``gdn_backward``  the gradients of ``gdn_forward``'s token rule by reverse-mode
  through the token loop, the state cotangent carried backwards (StateFlow
  Section 2.2, Eq. (6)-(7)).
* ``chunked_forward``  StateFlow Section 2.2 Eq. (2) chunk split, used only to
  check that the chunk algebra reproduces the token recurrence.
* ``forward_f32``   the token loops of ``gdn_forward`` / ``gla_forward`` in float32:
  the CPU throughput baseline of bench.py, never a parity reference.
* ``gdn_decode``    attention-gym "Linear Attention", the ``recurrent_gdn_decode``
  entry and the section "Gate Transforms" (``decode.py``, numpy float64).
* ``gdn_recurrent_paged``  the ``recurrent_gdn`` entry with a paged state pool:
  slot gather and scatter around ``gdn_forward`` (``decode.py``).
* ``gate_transform``  the section "Gate Transforms": both kinds, per-head and
  per-channel gates (``decode.py``).
* ``kda_forward``   the section "Kimi Delta Attention": the token rule with a
  per-channel decay (``decode.py``, numpy float64).
* ``kda_decode``    the ``recurrent_kda_decode`` entry (``decode.py``).

Pins: tests/test_oracle.py checks every function against closed forms,
brute-force products or invariants that do not reuse this code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE arithmetic, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
             "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.orc_gdn_forward.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, P, I]
        lib.orc_gla_forward.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, P, I]
        lib.orc_gdn_summary.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, P, P, I]
        lib.orc_gla_summary.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P, P, I]
        lib.orc_state_scan.argtypes = [I, P, P, P, I, I, I, I, I, P, P]
        lib.orc_chunked_forward.argtypes = [I, I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, P, I]
        lib.orc_forward_f32.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, I, I, I, ctypes.c_float, P, P, I]
        lib.orc_gdn_backward.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, D, P, P, P, P, P, P, I]
        lib.orc_gdn_backward.restype = None
        lib.orc_forward_f32.restype = None
        lib.orc_max_threads.restype = I
        for f in (lib.orc_gdn_forward, lib.orc_gla_forward, lib.orc_gdn_summary,
                  lib.orc_gla_summary, lib.orc_state_scan, lib.orc_chunked_forward):
            f.restype = None
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().orc_max_threads())


def _f32(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dims(q, v, cu_seqlens):
    B, T, HK, K = q.shape
    H, V = v.shape[2], v.shape[3]
    if cu_seqlens is None:
        cu = None
        N = B
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
        assert B == 1, "cu_seqlens needs batch-one inputs"
        assert cu[0] == 0 and np.all(np.diff(cu) >= 0) and cu[-1] <= T
    assert H % HK == 0
    return B, T, H, HK, K, V, N, cu


def gdn_forward(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, threads=0):
    """Token-by-token Gated Delta Rule. Returns (out [B,T,H,V], ht [N,H,V,K]) in float64.

    Output rows outside every sequence are NaN (they are never defined)."""
    q, k, v, g, beta, h0 = map(_f32, (q, k, v, g, beta, h0))
    B, T, H, HK, K, V, N, cu = _dims(q, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    out = np.full((B, T, H, V), np.nan, dtype=np.float64)
    ht = np.zeros((N, H, V, K), dtype=np.float64)
    _load().orc_gdn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                            _ptr(cu), N, B, T, H, HK, K, V, float(scale), _ptr(out),
                            _ptr(ht), int(threads))
    return out, ht


def gdn_backward(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None, scale=None, threads=0):
    """Gradients of the token-by-token Gated Delta Rule (reverse-mode through the token loop).

    do [B,T,H,V] and dht [N,H,V,K] (None: zero) are the upstream gradients of the outputs and final
    states. Returns a dict of float64 arrays dq, dk [B,T,HK,K] (summed over the value heads of each q/k
    head), dv [B,T,H,V], dg, dbeta [B,T,H], dh0 [N,H,V,K]. Entries of tokens outside every sequence are
    NaN."""
    q, k, v, g, beta, do, h0, dht = map(_f32, (q, k, v, g, beta, do, h0, dht))
    B, T, H, HK, K, V, N, cu = _dims(q, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    r = dict(dq=np.full((B, T, HK, K), np.nan), dk=np.full((B, T, HK, K), np.nan),
             dv=np.full((B, T, H, V), np.nan), dg=np.full((B, T, H), np.nan),
             dbeta=np.full((B, T, H), np.nan), dh0=np.zeros((N, H, V, K)))
    _load().orc_gdn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dht),
                             _ptr(cu), N, B, T, H, HK, K, V, float(scale), _ptr(r["dq"]), _ptr(r["dk"]),
                             _ptr(r["dv"]), _ptr(r["dg"]), _ptr(r["dbeta"]), _ptr(r["dh0"]), int(threads))
    return r


def gla_forward(q, k, v, g, h0=None, cu_seqlens=None, scale=1.0, threads=0):
    """Token-by-token scalar-gated linear attention. Returns (out, ht) in float64."""
    q, k, v, g, h0 = map(_f32, (q, k, v, g, h0))
    B, T, H, HK, K, V, N, cu = _dims(q, v, cu_seqlens)
    out = np.full((B, T, H, V), np.nan, dtype=np.float64)
    ht = np.zeros((N, H, V, K), dtype=np.float64)
    _load().orc_gla_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(h0), _ptr(cu),
                            N, B, T, H, HK, K, V, float(scale), _ptr(out), _ptr(ht),
                            int(threads))
    return out, ht


def forward_f32(kind, q, k, v, g, beta=None, h0=None, cu_seqlens=None, scale=None, threads=0):
    """Float32 build of the token loops (kind "gdn" or "gla"): the same steps as gdn_forward /
    gla_forward in float arithmetic. CPU throughput baseline only, never a parity reference.
    Returns (out, ht) in float32."""
    q, k, v, g, beta, h0 = map(_f32, (q, k, v, g, beta, h0))
    B, T, H, HK, K, V, N, cu = _dims(q, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / np.sqrt(K) if kind == "gdn" else 1.0
    out = np.full((B, T, H, V), np.nan, dtype=np.float32)
    ht = np.zeros((N, H, V, K), dtype=np.float32)
    _load().orc_forward_f32(1 if kind == "gdn" else 0, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                            _ptr(h0), _ptr(cu), N, B, T, H, HK, K, V, float(scale), _ptr(out), _ptr(ht),
                            int(threads))
    return out, ht


def gdn_summary(k, v, g, beta, cu_seqlens=None, threads=0):
    """Affine summary of each range: exit = entry @ M + S_ext. Returns (M [N,H,K,K], S_ext [N,H,V,K])."""
    k, v, g, beta = map(_f32, (k, v, g, beta))
    B, T, H, HK, K, V, N, cu = _dims(k, v, cu_seqlens)
    M = np.zeros((N, H, K, K), dtype=np.float64)
    S_ext = np.zeros((N, H, V, K), dtype=np.float64)
    _load().orc_gdn_summary(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu), N, B, T,
                            H, HK, K, V, _ptr(M), _ptr(S_ext), int(threads))
    return M, S_ext


def gla_summary(k, v, g, cu_seqlens=None, threads=0):
    """Scalar-gate summary: exit = a * entry + S_ext. Returns (a [N,H], S_ext [N,H,V,K])."""
    k, v, g = map(_f32, (k, v, g))
    B, T, H, HK, K, V, N, cu = _dims(k, v, cu_seqlens)
    a = np.zeros((N, H), dtype=np.float64)
    S_ext = np.zeros((N, H, V, K), dtype=np.float64)
    _load().orc_gla_summary(_ptr(k), _ptr(v), _ptr(g), _ptr(cu), N, B, T, H, HK, K, V,
                            _ptr(a), _ptr(S_ext), int(threads))
    return a, S_ext


def state_scan(kind, M, S_ext, h0=None, *, B, n_seg):
    """Exclusive scan over segment rows s = b*n_seg + j.

    kind "gdn": M [B*n_seg, H, K, K]; kind "gla": M is a [B*n_seg, H].
    Returns (S_in [B*n_seg, H, V, K], S_final [B, H, V, K])."""
    M, S_ext, h0 = map(_f64, (M, S_ext, h0))
    rows, H, V, K = S_ext.shape
    assert rows == B * n_seg
    S_in = np.zeros_like(S_ext)
    S_final = np.zeros((B, H, V, K), dtype=np.float64)
    _load().orc_state_scan(0 if kind == "gdn" else 1, _ptr(M), _ptr(S_ext), _ptr(h0), B,
                           n_seg, H, K, V, _ptr(S_in), _ptr(S_final))
    return S_in, S_final


def chunked_forward(kind, q, k, v, g, beta=None, h0=None, cu_seqlens=None, scale=None,
                    chunk=64, threads=0):
    """Chunked form (self-check of the chunk algebra only). kind: "gdn" or "gla"."""
    q, k, v, g, beta, h0 = map(_f32, (q, k, v, g, beta, h0))
    B, T, H, HK, K, V, N, cu = _dims(q, v, cu_seqlens)
    if scale is None:
        scale = 1.0 / np.sqrt(K) if kind == "gdn" else 1.0
    out = np.full((B, T, H, V), np.nan, dtype=np.float64)
    ht = np.zeros((N, H, V, K), dtype=np.float64)
    _load().orc_chunked_forward(1 if kind == "gdn" else 0, int(chunk), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(cu), N, B, T,
                                H, HK, K, V, float(scale), _ptr(out), _ptr(ht), int(threads))
    return out, ht


from .decode import gate_transform, gdn_decode, gdn_recurrent_paged, kda_decode, kda_forward  # noqa: E402  (numpy float64, no C part)

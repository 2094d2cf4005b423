"""Seeded synthetic inputs for the chunked linear recurrence (no method arithmetic).

This module only draws random tensors. It is the one piece of code that both
the oracle tests and the GPU path use, so it holds nothing of the recurrence
itself: no decay, no state, no output. Every tensor is drawn in float32 on the
CPU from numpy's PCG64 generator and, where the workload is bf16, cast once
with torch (round to nearest even); both sides then receive exactly the same
values (the oracle widens them to float64 exactly).

The five named workloads follow the statement of the problem (shapes, value
distributions, chunk sizes, segment counts), with the readings taken where it
is open noted in the workload functions below:

1. ``tiny_gdn``       B=1 T=256 H=2 K=V=64, float32, chunk 64.
2. ``dense_gdn``      B=2 T=4096 H=16 K=V=128, bf16, initial state N(0, 0.02).
3. ``varlen_gdn``     batch-one packed stream of 32768 tokens, 9 sequences
                      (one empty, tails), H=32 K=V=128, bf16.
4. ``long_gdn``       B=1 T=262144 H=16 K=V=128, bf16, 16 segments of 16384.
5. ``ssd_gla``        scalar-gate linear attention, B=2 T=16384 H=64 HK=8,
                      K=128 (dstate), V=64 (headdim), chunk 128, 8 segments per row.

and one decode workload (one token per sequence against a paged state pool):

6. ``decode_gdn``     B=256 sequences, H=HK=32, K=V=128 (the packed workload's
                      heads), bf16 packed [Q | K | V] rows, float32 pool of 257
                      slots (slot 0 the null slot), every row active.
7. ``recurrent_gdn``  64 sequences of 16 tokens, H=HK=32, K=V=128, bf16, on a
                      float32 pool of 65 slots (token-by-token forward).
8. ``gate_transform`` per-channel raw gates [2, 16384, 16, 128] bf16, softplus kind.
9. ``paged_gdn``      the packed workload's stream on a float32 state pool (chunk
                      forward advancing the cache in place).
10. ``recurrent_kda`` recurrent_gdn's shapes with a per-channel gate (Kimi Delta
                      Attention token by token).
11. ``decode_kda``    decode_gdn's shapes for the KDA decode (per-channel raw gates,
                      bounded kind with lower bound -5).

Draw order inside one workload: q, k, v, gate noise, beta noise, h0, A, dt,
sequence lengths.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

SEEDS = {"tiny_gdn": 101, "dense_gdn": 102, "varlen_gdn": 103, "long_gdn": 104, "ssd_gla": 105,
         "decode_gdn": 106, "recurrent_gdn": 107, "gate_transform": 108,
         "paged_gdn": 109, "recurrent_kda": 110, "decode_kda": 111, "dense_gdn_bwd": 112, "dense_kda": 113}


@dataclass
class Workload:
    name: str
    kind: str                      # "gdn" or "gla"
    q: torch.Tensor                # [B, T, HK, K]
    k: torch.Tensor                # [B, T, HK, K]
    v: torch.Tensor                # [B, T, H, V]
    g: torch.Tensor                # [B, T, H] float32, natural-log gate
    beta: Optional[torch.Tensor]   # [B, T, H] float32 (delta rule only)
    h0: Optional[torch.Tensor]     # [N, H, V, K] float32 or None
    cu_seqlens: Optional[torch.Tensor]  # int32 [N + 1] or None
    scale: float
    chunk: int
    n_seg: int = 1                 # segments per batch row (1 = unsegmented)
    meta: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        return self.q.shape[1]

    @property
    def H(self):
        return self.v.shape[2]

    @property
    def HK(self):
        return self.q.shape[2]

    @property
    def K(self):
        return self.q.shape[3]

    @property
    def V(self):
        return self.v.shape[3]

    @property
    def N(self):
        return self.B if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    @property
    def tokens(self) -> int:
        """Active tokens (per the packed offsets when present)."""
        if self.cu_seqlens is None:
            return self.B * self.T
        return int(self.cu_seqlens[-1])


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _l2rows(x):
    # unit rows over the last axis, in float32, no epsilon (N(0,1) rows are never zero)
    return (x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))).astype(np.float32)


def _softplus(x):
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _cast(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype) if dtype != torch.float32 else t


def delta_rule_inputs(*, B, T, H, K, V, HK=None, dtype=torch.bfloat16, seed=0,
                      gate_shift=0.0, h0_std=None, N=None, normalize_qk=True,
                      beta_scale=1.0):
    """q, k (unit rows), v ~ N(0,1); g = -softplus(N(0,1) + gate_shift); beta = sigmoid(N(0,1))."""
    HK = HK or H
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, T, HK, K))
    k = _normal(rng, (B, T, HK, K))
    if normalize_qk:
        q, k = _l2rows(q), _l2rows(k)
    v = _normal(rng, (B, T, H, V))
    g = -_softplus(_normal(rng, (B, T, H)) + np.float32(gate_shift))
    beta = (_sigmoid(_normal(rng, (B, T, H))) * np.float32(beta_scale)).astype(np.float32)
    h0 = None
    if h0_std is not None:
        h0 = torch.from_numpy(_normal(rng, (N or B, H, V, K)) * np.float32(h0_std))
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype),
                g=torch.from_numpy(g), beta=torch.from_numpy(beta), h0=h0, rng=rng)


def upstream_grads(rng, *, B, T, H, V, K, N, dtype=torch.bfloat16, dht=True):
    """Upstream gradients for the backward: do ~ N(0,1) [B,T,H,V] in the input type, dht ~ N(0,1) float32
    [N,H,V,K] (or None)."""
    do = _normal(rng, (B, T, H, V))
    dh = torch.from_numpy(_normal(rng, (N, H, V, K))) if dht else None
    return dict(do=_cast(do, dtype), dht=dh)


def scalar_gate_inputs(*, B, T, H, HK, K, V, dtype=torch.bfloat16, seed=0):
    """q, k, v ~ N(0,1) (not normalised); per-head A = -softplus(N(0,1)) [H];
    dt = softplus(N(0,1)) [B, T, H]; g = A * dt."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, T, HK, K))
    k = _normal(rng, (B, T, HK, K))
    v = _normal(rng, (B, T, H, V))
    A = -_softplus(_normal(rng, (H,)))
    dt = _softplus(_normal(rng, (B, T, H)))
    g = (A[None, None, :] * dt).astype(np.float32)
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype),
                g=torch.from_numpy(g), A=A, rng=rng)


def varlen_lengths(rng, total, n_long=7, min_ragged=3, chunk=64):
    """Sequence lengths of the packed workload: one short sequence (1..63 tokens),
    n_long more from distinct random cuts, then one empty sequence at a random slot.
    All lengths sum to ``total``; at least ``min_ragged`` of the nonempty ones are
    not multiples of ``chunk``."""
    short = int(rng.integers(1, chunk))
    while True:
        cuts = np.sort(rng.choice(np.arange(1, total - short), size=n_long - 1, replace=False))
        edges = np.concatenate([[0], cuts, [total - short]])
        longs = np.diff(edges).astype(np.int64)
        lens = np.concatenate([[short], longs])
        if np.count_nonzero(lens % chunk) >= min_ragged and np.all(lens > 0):
            break
    rng.shuffle(lens)
    pos = int(rng.integers(0, len(lens) + 1))
    lens = np.insert(lens, pos, 0)
    assert lens.sum() == total
    return lens


def cu_from_lengths(lens):
    return torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))


def tiny_gdn(seed=SEEDS["tiny_gdn"]):
    """float32 delta rule; scale 1/sqrt(64) = 1/8, zero initial state."""
    d = delta_rule_inputs(B=1, T=256, H=2, K=64, V=64, dtype=torch.float32, seed=seed)
    return Workload("tiny_gdn", "gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], None, None,
                    scale=1.0 / 8.0, chunk=64)


def dense_gdn(seed=SEEDS["dense_gdn"], *, B=2, T=4096, H=16, D=128):
    """bf16 delta rule; g = -softplus(N(0,1) + 2); initial state N(0, 0.02) read as standard deviation
    0.02; scale 1/sqrt(D)."""
    d = delta_rule_inputs(B=B, T=T, H=H, K=D, V=D, dtype=torch.bfloat16, seed=seed,
                          gate_shift=2.0, h0_std=0.02)
    return Workload("dense_gdn", "gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None,
                    scale=1.0 / np.sqrt(D), chunk=64)


def dense_gdn_bwd(seed=SEEDS["dense_gdn_bwd"], *, B=2, T=4096, H=16, D=128):
    """The dense prefill inputs (dense_gdn's generator and seed) and, for the backward, upstream gradients
    do ~ N(0,1) (bf16) and dht ~ N(0,1) (float32) drawn with this seed."""
    w = dense_gdn(B=B, T=T, H=H, D=D)
    u = upstream_grads(np.random.default_rng(seed), B=B, T=T, H=H, V=D, K=D, N=B)
    w.name = "dense_gdn_bwd"
    w.meta.update(do=u["do"], dht=u["dht"])
    return w


def varlen_gdn(seed=SEEDS["varlen_gdn"], *, T=32768, H=32, D=128, n_long=7):
    """bf16 delta rule on one packed stream; lengths from varlen_lengths (one short length, the others
    from random cuts with at least three not multiples of 64, one empty sequence inserted); gates and
    distributions as dense_gdn; zero initial states."""
    d = delta_rule_inputs(B=1, T=T, H=H, K=D, V=D, dtype=torch.bfloat16, seed=seed, gate_shift=2.0)
    lens = varlen_lengths(d["rng"], T, n_long=n_long)
    return Workload("varlen_gdn", "gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], None,
                    cu_from_lengths(lens), scale=1.0 / np.sqrt(D), chunk=64,
                    meta={"lengths": [int(x) for x in lens]})


def paged_gdn(seed=SEEDS["paged_gdn"], *, T=32768, H=32, D=128, n_long=7):
    """varlen_gdn's stream and distributions, each sequence starting from its slot of a float32 pool
    (N + 1 slots, every sequence loaded; pool ~ N(0, 0.02^2), slots a random permutation of 1..N)."""
    w = varlen_gdn(seed=seed, T=T, H=H, D=D, n_long=n_long)
    rng = np.random.default_rng(seed + 1000)
    N = w.N
    pool = _normal(rng, (N + 1, H, D, D)) * np.float32(0.02)
    idx = rng.permutation(np.arange(1, N + 1)).astype(np.int32)
    w.name = "paged_gdn"
    w.meta.update(pool=torch.from_numpy(pool), state_indices=torch.from_numpy(idx))
    return w


def kda_inputs(*, B, T, H, K, V, dtype=torch.bfloat16, seed=0, gate_shift=2.0, h0_std=None, N=None):
    """q, k (unit rows), v ~ N(0,1); per-channel g = -softplus(N(0,1) + gate_shift) [B, T, H, K];
    beta = sigmoid(N(0,1))."""
    rng = np.random.default_rng(seed)
    q = _l2rows(_normal(rng, (B, T, H, K)))
    k = _l2rows(_normal(rng, (B, T, H, K)))
    v = _normal(rng, (B, T, H, V))
    g = -_softplus(_normal(rng, (B, T, H, K)) + np.float32(gate_shift))
    beta = _sigmoid(_normal(rng, (B, T, H)))
    h0 = None if h0_std is None else torch.from_numpy(_normal(rng, (N or B, H, V, K)) * np.float32(h0_std))
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), g=torch.from_numpy(g),
                beta=torch.from_numpy(beta), h0=h0, rng=rng)


def dense_kda(seed=SEEDS["dense_kda"], *, B=2, T=4096, H=16, D=128):
    """KDA chunk prefill at the dense prefill shape: q, k (unit rows), v ~ N(0,1) bf16; per-channel
    g = -softplus(N(0,1) + 2) float32 [B, T, H, D]; beta = sigmoid(N(0,1)); initial state N(0, 0.02);
    scale 1/sqrt(D)."""
    d = kda_inputs(B=B, T=T, H=H, K=D, V=D, seed=seed, h0_std=0.02)
    return Workload("dense_kda", "kda", d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None,
                    scale=1.0 / np.sqrt(D), chunk=64)


def recurrent_kda(seed=SEEDS["recurrent_kda"], *, B=64, T=16, H=32, D=128):
    """recurrent_gdn's shapes and pool with a per-channel gate (a reading, as there)."""
    d = kda_inputs(B=B, T=T, H=H, K=D, V=D, seed=seed)
    rng = d["rng"]
    pool = _normal(rng, (B + 1, H, D, D)) * np.float32(0.02)
    idx = rng.permutation(np.arange(1, B + 1)).astype(np.int32)
    return Workload("recurrent_kda", "kda", d["q"], d["k"], d["v"], d["g"], d["beta"], None, None,
                    scale=1.0 / np.sqrt(D), chunk=0,
                    meta={"pool": torch.from_numpy(pool), "state_indices": torch.from_numpy(idx)})


def long_gdn(seed=SEEDS["long_gdn"], *, T=262144, H=16, D=128, n_seg=16):
    """bf16 delta rule on one long row cut into n_seg segments; g = -softplus(N(0,1) + 4) as the
    formula gives it (its decay is fast, whatever the label says); zero initial state; scale 1/sqrt(D)."""
    d = delta_rule_inputs(B=1, T=T, H=H, K=D, V=D, dtype=torch.bfloat16, seed=seed, gate_shift=4.0)
    return Workload("long_gdn", "gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], None, None,
                    scale=1.0 / np.sqrt(D), chunk=64, n_seg=n_seg)


def ssd_gla(seed=SEEDS["ssd_gla"], *, B=2, T=16384, H=64, HK=8, K=128, V=64, n_seg=8):
    """bf16 scalar-gated recurrence; A = -softplus(N(0,1)) once per head, dt = softplus(N(0,1)) per
    token, g = A dt; q, k, v ~ N(0,1) unnormalised and v used as given; zero initial state; scale 1."""
    d = scalar_gate_inputs(B=B, T=T, H=H, HK=HK, K=K, V=V, seed=seed)
    return Workload("ssd_gla", "gla", d["q"], d["k"], d["v"], d["g"], None, None, None,
                    scale=1.0, chunk=128, n_seg=n_seg, meta={"A": d["A"]})


@dataclass
class DecodeWorkload:
    name: str
    packed_qkv: torch.Tensor       # [B, 2*HK*K + H*V]: query heads, key heads, value heads
    raw_gate: torch.Tensor         # [1, B, H], element type of packed_qkv
    raw_beta: torch.Tensor         # [1, B, H]
    A_log: torch.Tensor            # [H] float32
    dt_bias: torch.Tensor          # [H] float32
    pool: torch.Tensor             # [num_slots, H, V, K] float32 or bf16
    state_indices: torch.Tensor    # [B] int32; <= 0 marks a null row
    has_initial_state: Optional[torch.Tensor]  # [B] bool or None (all loaded)
    H: int
    HK: int
    K: int
    V: int
    scale: float
    per_channel: bool = False          # Kimi Delta Attention: raw_gate [1, B, H, K], dt_bias [H, K]
    gate_kind: str = "softplus"
    lower_bound: Optional[float] = None

    @property
    def B(self):
        return self.packed_qkv.shape[0]

    @property
    def tokens(self) -> int:
        """Rows that advance a slot (one token each)."""
        return int((self.state_indices > 0).sum())


def decode_inputs(*, B, H, HK, K, V, dtype=torch.bfloat16, pool_dtype=torch.float32, seed=0,
                  num_slots=None, n_null=0, n_fresh=0, pool_std=0.02):
    """packed rows, raw gate and raw beta ~ N(0,1); A_log = log U(1, 16) per head; dt_bias ~
    N(-3, 1) per head; pool ~ N(0, pool_std^2); slots a random permutation of 1..num_slots-1, then
    n_null rows set to the null indices 0 and -1 (alternating) and n_fresh other rows marked fresh."""
    rng = np.random.default_rng(seed)
    num_slots = num_slots or B + 1
    assert num_slots - 1 >= B and n_null + n_fresh <= B
    packed = _normal(rng, (B, 2 * HK * K + H * V))
    raw_gate = _normal(rng, (1, B, H))
    raw_beta = _normal(rng, (1, B, H))
    A_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = (rng.standard_normal(H) - 3.0).astype(np.float32)
    pool = _normal(rng, (num_slots, H, V, K)) * np.float32(pool_std)
    idx = rng.permutation(np.arange(1, num_slots))[:B].astype(np.int32)
    rows = rng.permutation(B)
    for i, r in enumerate(rows[:n_null]):
        idx[r] = 0 if i % 2 == 0 else -1
    fresh = None
    if n_fresh:
        fresh = np.ones(B, dtype=bool)
        fresh[rows[n_null:n_null + n_fresh]] = False
    return dict(packed_qkv=_cast(packed, dtype), raw_gate=_cast(raw_gate, dtype), raw_beta=_cast(raw_beta, dtype),
                A_log=torch.from_numpy(A_log), dt_bias=torch.from_numpy(dt_bias), pool=_cast(pool, pool_dtype),
                state_indices=torch.from_numpy(idx),
                has_initial_state=None if fresh is None else torch.from_numpy(fresh))


def kda_decode_inputs(*, B, H, K, V, dtype=torch.bfloat16, pool_dtype=torch.float32, seed=0, **kw):
    """decode_inputs with HK = H, then per-channel raw gates ~ N(0,1) [1, B, H, K] and dt_bias ~
    N(0, 1) [H, K] (drawn after the rest)."""
    d = decode_inputs(B=B, H=H, HK=H, K=K, V=V, dtype=dtype, pool_dtype=pool_dtype, seed=seed, **kw)
    rng = np.random.default_rng(seed + 7919)
    d["raw_gate"] = _cast(_normal(rng, (1, B, H, K)), dtype)
    d["dt_bias"] = torch.from_numpy(rng.standard_normal((H, K)).astype(np.float32))
    return d


def decode_kda(seed=SEEDS["decode_kda"], *, B=256, H=32, D=128):
    """decode_gdn's shapes for the KDA decode, bounded kind with the entry's default lower bound -5."""
    d = kda_decode_inputs(B=B, H=H, K=D, V=D, seed=seed)
    return DecodeWorkload("decode_kda", H=H, HK=H, K=D, V=D, scale=1.0 / np.sqrt(D), per_channel=True,
                          gate_kind="bounded", lower_bound=-5.0, **d)


def decode_gdn(seed=SEEDS["decode_gdn"], *, B=256, H=32, HK=32, D=128):
    """One decode token for each of B sequences; every row active and loaded; scale 1/sqrt(D). The
    pages give no decode batch: 256 rows of the packed workload's heads is the reading taken."""
    d = decode_inputs(B=B, H=H, HK=HK, K=D, V=D, seed=seed)
    return DecodeWorkload("decode_gdn", H=H, HK=HK, K=D, V=D, scale=1.0 / np.sqrt(D), **d)


def recurrent_gdn(seed=SEEDS["recurrent_gdn"], *, B=64, T=16, H=32, D=128):
    """A short multi-token step for each of B sequences on a paged float32 pool (B + 1 slots, every
    sequence loaded): q, k unit rows, v ~ N(0,1), g and beta as dense_gdn, pool ~ N(0, 0.02^2), slots
    a random permutation of 1..B. The pages give no such batch: 64 sequences of 16 tokens with the
    packed workload's heads is the reading taken."""
    d = delta_rule_inputs(B=B, T=T, H=H, K=D, V=D, dtype=torch.bfloat16, seed=seed, gate_shift=2.0)
    rng = d["rng"]
    pool = _normal(rng, (B + 1, H, D, D)) * np.float32(0.02)
    idx = rng.permutation(np.arange(1, B + 1)).astype(np.int32)
    return Workload("recurrent_gdn", "gdn", d["q"], d["k"], d["v"], d["g"], d["beta"], None, None,
                    scale=1.0 / np.sqrt(D), chunk=0,
                    meta={"pool": torch.from_numpy(pool), "state_indices": torch.from_numpy(idx)})


@dataclass
class GateWorkload:
    name: str
    raw: torch.Tensor       # [..., H] or [..., H, D]
    A_log: torch.Tensor     # [H] float32
    dt_bias: torch.Tensor   # [H] or [H, D] float32
    kind: str
    lower_bound: Optional[float] = None

    @property
    def tokens(self) -> int:
        return int(np.prod(self.raw.shape[:-2 if self.dt_bias.dim() == 2 else -1]))


def gate_inputs(*, shape, H, D=None, dtype=torch.bfloat16, seed=0):
    """raw ~ N(0,1) of the given shape; A_log = log U(1, 16) per head; dt_bias ~ N(-3, 1) per head
    (or per head and channel)."""
    rng = np.random.default_rng(seed)
    raw = _normal(rng, shape)
    A_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = (rng.standard_normal(H if D is None else (H, D)) - 3.0).astype(np.float32)
    return dict(raw=_cast(raw, dtype), A_log=torch.from_numpy(A_log), dt_bias=torch.from_numpy(dt_bias))


def gate_transform(seed=SEEDS["gate_transform"], *, B=2, T=16384, H=16, D=128):
    """Per-channel raw gates of a long bf16 batch through the softplus kind. The pages give no
    standalone size for this step: the long scalar-gate batch's token count with the dense
    workload's heads and head width is the reading taken."""
    d = gate_inputs(shape=(B, T, H, D), H=H, D=D, seed=seed)
    return GateWorkload("gate_transform", kind="softplus", **d)


CONFIGS = {"tiny_gdn": tiny_gdn, "dense_gdn": dense_gdn, "varlen_gdn": varlen_gdn,
           "long_gdn": long_gdn, "ssd_gla": ssd_gla, "decode_gdn": decode_gdn,
           "recurrent_gdn": recurrent_gdn, "gate_transform": gate_transform,
           "paged_gdn": paged_gdn, "recurrent_kda": recurrent_kda, "decode_kda": decode_kda,
           "dense_gdn_bwd": dense_gdn_bwd, "dense_kda": dense_kda}


def to_f32(t):
    """Exact float32 numpy copy of a CPU tensor (bf16 widens exactly)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float32).numpy()

#!/usr/bin/env python3
"""Throughput of the Gated Delta Rule chunk forward on one MI355X.

Workload (default): dense GDN prefill, B=2, T=4096, H=16, K=V=128, bf16 q/k/v,
float32 gate/beta/state, chunk 64, initial state N(0, 0.02) -- the configuration
the headline metric is quoted on. One step is one full sf_gdn_chunk_fwd call
(gate cumsum, K K^T / Q K^T, triangular solve, state transition, output, final
state) on one batch of seeded synthetic inputs already resident in HBM. Several
input sets (--rotate, default 3, 310 MB > the 256 MB last-level cache) are
cycled so consecutive steps cannot be served from the cache.

Prints one JSON line with tokens/s (from the timed steps as a caller runs them),
the roofline fraction of the dominant kernel (its average launch time from HIP
events recorded on the launch stream around every launch, in a second timed
pass over the same steps; the events add gaps between launches, so that pass's
step time is reported apart as events_pass_ms_per_step), p50_ms and min_ms of the
per-step times (one event between consecutive steps on the launch stream), and the
oracle's float32 token loops timed on the host cores on the same workload
(cpu_baseline, with the core count and CPU model; a reported baseline, not a
target). Segmented workloads also carry path_roofline_two_pass, the path's
fraction on the byte count of the summary-scan-finalize method. Beside the published HBM peak, the roofline objects
carry measured_peak: the bandwidth a plain 1 GiB device-to-device copy reaches
on the same GPU (read plus write bytes), and the fraction of that.

Other workloads (--workload varlen_gdn | long_gdn | ssd_gla | tiny_gdn | decode_gdn | recurrent_gdn |
gate_transform | paged_gdn | recurrent_kda | decode_kda | dense_gdn_bwd | dense_kda) are for
measurement only; the headline line is the default one. decode_gdn times one sf_gdn_decode call
(one token for each of 256 sequences against a 514 MB float32 state pool, which is larger than
the last-level cache, so it runs on one input set).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunk-fwd tokens/s (bf16, K=V=128) + % of MFMA/HBM roofline, 1 MI355X"
METRIC_BWD = "GDN chunk-bwd tokens/s (bf16, K=V=128) + % of roofline, 1 MI355X"
METRIC_KDA = "KDA chunk-fwd tokens/s (bf16, K=V=128) + % of HBM roofline, 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3        # MI355X dense float32 MFMA, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(w):
    """One decode step: every active row reads (unless fresh) and writes its H states of V*K pool
    elements, reads its packed row and its 2 H raw gates, writes H*V outputs; A_log and dt_bias."""
    import torch
    eb = w.packed_qkv.element_size()
    pe = w.pool.element_size()
    active = w.state_indices > 0
    loaded = active if w.has_initial_state is None else active & w.has_initial_state
    states = (int(active.sum()) + int(loaded.sum())) * w.H * w.V * w.K * pe
    rows = (w.packed_qkv.numel() + w.raw_gate.numel() + w.raw_beta.numel()) * eb + w.B * w.H * w.V * eb
    return states + rows + (w.A_log.numel() + w.dt_bias.numel()) * 4 + w.B * 4


def algorithmic_bytes(w, kernel):
    """Bytes a kernel must move by definition of the computation (no intermediates).

    Delta rule, per token and value head: q, k, v and o in the element type
    (HK/H of q and k per value head), plus gate and beta in float32; per
    (sequence, head): the initial state read (when given) and the final state
    written, V*K float32 each."""
    if kernel in ("gdn_decode", "kda_decode", "decode_path"):
        return decode_bytes(w)
    if w.name == "dense_gdn_bwd":
        return bwd_bytes(w, kernel)
    if kernel in ("gate_transform", "gate_path"):   # raw in, float32 out, the per-head parameters
        return w.raw.numel() * (w.raw.element_size() + 4) + (w.A_log.numel() + w.dt_bias.numel()) * 4
    eb = w.q.element_size()
    tok = w.tokens
    qk = 2 * tok * w.HK * w.K * eb
    vo = 2 * tok * w.H * w.V * eb
    gb = tok * w.H * 4 * (2 if w.beta is not None else 1)
    states = w.N * w.H * w.V * w.K * 4 * (1 + (w.h0 is not None))
    if w.name in ("recurrent_kda", "dense_kda"):   # per-channel gate: K floats per token and head
        gb = tok * w.H * 4 * (w.K + 1)
    if w.name == "dense_kda":
        # kda_prep reads q, k, v, g, beta; kda_chain reads h0 and writes o and ht
        if kernel == "kda_prep":
            return qk + vo // 2 + gb
        if kernel == "kda_chain":
            return vo // 2 + states
    if kernel == "gdn_prep":                      # Pre reads k, the gate and beta
        return qk // 2 + gb
    if kernel == "gdn_summary_chain":             # k, v in; each segment's M [K][K] and S_ext [V][K] out
        return qk // 2 + vo // 2 + w.B * w.n_seg * w.H * (w.K * w.K + w.V * w.K) * 4
    if w.name in ("recurrent_gdn", "paged_gdn", "recurrent_kda"):   # every slot read and written (float32 pool)
        states = 2 * w.N * w.H * w.V * w.K * w.meta["pool"].element_size()
        return qk + vo + states + (0 if kernel in ("gdn_chain", "gdn_chain_slice") else gb)
    if kernel in ("gdn_chain", "gdn_chain_slice", "gla_chain"):
        return qk + vo + states
    return qk + vo + gb + states      # whole path


def bwd_bytes(w, kernel):
    """Chunk backward, by definition of the computation: reads q, k, v, do (element type), g and beta
    (float32), h0 and dht; writes dq, dk, dv (element type), dg and dbeta (float32) and dh0. Per kernel,
    the share each one reads or writes of those (its intermediates excluded)."""
    eb = w.q.element_size()
    tok = w.tokens
    row = tok * w.H * w.K * eb            # one of q, k, v, do, dq, dk, dv (K == V)
    gate = tok * w.H * 4                  # one of g, beta, dg, dbeta
    state = w.N * w.H * w.V * w.K * 4     # one of h0, dht, dh0
    parts = {"gdn_bwd_prep": 2 * row + 2 * gate,          # q, k, g, beta
             "gdn_bwd_states": 2 * row + state,           # k, v, h0
             "gdn_bwd_dstate": 2 * row + 2 * state,       # k, do, dht, dh0
             "gdn_bwd_grad": 4 * row + 3 * row + 2 * gate}  # q, k, v, do; dq, dk, dv, dg, dbeta
    if kernel in parts:
        return parts[kernel]
    return 7 * row + 4 * gate + 3 * state


def bwd_grad_flops(w):
    """Contraction flops the chunk backward's per-chunk gradients need (2 per multiply-add), by the
    formulas of the chunk backward, triangular factors counted on their lower-triangular pairs only:
    X, Q S, K dS', dO S, dX S, R dS' (C K V each); Q K^T, K K^T, dP K, dP^T Q, dT K, dT^T K (C(C+1)/2 K
    each); T Z, P^T dO, T^T dR, dO R^T, dR Z^T (C(C+1)/2 V each); dT T and the dA product (C^3/6 each)."""
    C = w.chunk
    c2 = C * (C + 1) // 2
    mac = 6 * C * w.K * w.V + 6 * c2 * w.K + 5 * c2 * w.V + C ** 3 // 3
    chunks = (w.tokens // C) * w.H
    return 2 * mac * chunks


def two_pass_bytes(w):
    """Bytes of the segmented method (summary pass, scan, finalize pass), for workloads cut into
    segments: pass 1 reads k, v, g (and beta) and writes every segment's summary (M or a_block, and
    S_ext); the scan reads the summaries and writes the entry states S_in; pass 2 is the whole path
    on the segment view with S_in read as its initial states. None for unsegmented workloads."""
    if not getattr(w, "n_seg", None) or w.n_seg <= 1:
        return None
    eb = w.q.element_size()
    tok = w.tokens
    rows = w.B * w.n_seg
    state = w.H * w.V * w.K * 4
    delta = w.beta is not None
    summ = rows * (state + (w.H * w.K * w.K * 4 if delta else w.H * 4))
    pass1 = tok * w.HK * w.K * eb + tok * w.H * w.V * eb + tok * w.H * 4 * (2 if delta else 1) + summ
    scan = summ + rows * state + w.B * state          # read summaries, write S_in and the final state
    pass2 = algorithmic_bytes(w, "path") + rows * state
    return pass1 + scan + pass2


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE (scaled by a copy-kernel
    calibration) from profiles/<kernel>_<workload>_traffic.txt, or None when absent or when the
    kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = os.path.join(ROOT, "chunked_linear_recurrence_amd", "csrc", kv.get("source", "gdn.hip"))
    if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != kv.get("source_sha256_16"):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_sets(w, dev, rotate):
    import torch
    import workloads as wl
    if isinstance(w, wl.GateWorkload):
        return [{n: getattr(w, n).to(dev).contiguous() for n in ("raw", "A_log", "dt_bias")} for _ in range(rotate)]
    if isinstance(w, wl.DecodeWorkload):
        s = {n: (None if getattr(w, n) is None else getattr(w, n).to(dev).contiguous())
             for n in ("packed_qkv", "raw_gate", "raw_beta", "A_log", "dt_bias", "pool", "state_indices",
                       "has_initial_state")}
        s["out"] = torch.empty((1, w.B, w.H, w.V), dtype=w.packed_qkv.dtype, device=dev)
        return [s]
    sets = []
    for r in range(rotate):
        s = {}
        for n in ("q", "k", "v", "g", "beta", "h0", "cu_seqlens"):
            t = getattr(w, n)
            s[n] = None if t is None else t.to(dev).contiguous()
        if w.name == "dense_gdn_bwd":
            s["do"] = w.meta["do"].to(dev).contiguous()
            s["dht"] = w.meta["dht"].to(dev).contiguous()
        if w.name in ("recurrent_gdn", "paged_gdn", "recurrent_kda"):
            s["pool"] = w.meta["pool"].to(dev).contiguous()
            s["state_indices"] = w.meta["state_indices"].to(dev)
        sets.append(s)
    return sets


def step_fn(w):
    import chunked_linear_recurrence_amd as sf
    if w.name == "gate_transform":
        def step(s):
            return sf.gate_transform(s["raw"], s["A_log"], s["dt_bias"], kind=w.kind, lower_bound=w.lower_bound)
    elif w.name == "decode_kda":
        def step(s):
            return sf.kda_decode(s["packed_qkv"], s["raw_gate"], s["raw_beta"], s["A_log"], s["dt_bias"], s["pool"],
                                 s["state_indices"], has_initial_state=s["has_initial_state"],
                                 gate_transform=w.gate_kind, lower_bound=w.lower_bound, scale=w.scale, out=s["out"])
    elif w.name == "decode_gdn":
        def step(s):
            return sf.gdn_decode(s["packed_qkv"], s["raw_gate"], s["raw_beta"], s["A_log"], s["dt_bias"], s["pool"],
                                 s["state_indices"], has_initial_state=s["has_initial_state"], scale=w.scale,
                                 out=s["out"])
    elif w.name == "paged_gdn":
        def step(s):
            return sf.paged_gdn_chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["pool"], s["state_indices"],
                                          cu_seqlens=s["cu_seqlens"], scale=w.scale)
    elif w.name == "recurrent_kda":
        def step(s):
            return sf.kda_recurrent_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["pool"],
                                        state_indices=s["state_indices"], scale=w.scale)
    elif w.name == "recurrent_gdn":
        def step(s):
            return sf.gdn_recurrent_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["pool"],
                                        state_indices=s["state_indices"], scale=w.scale)
    elif w.name == "dense_gdn_bwd":
        def step(s):
            return sf.gdn_chunk_bwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["do"], s["h0"], s["dht"],
                                    scale=w.scale)
    elif w.name == "dense_kda":
        def step(s):
            return sf.kda_chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["h0"], scale=w.scale,
                                    output_final_state=True)
    elif w.name in ("dense_gdn", "tiny_gdn", "varlen_gdn"):
        def step(s):
            return sf.gdn_chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["h0"], cu_seqlens=s["cu_seqlens"],
                                    scale=w.scale, output_final_state=True)
    elif w.name == "long_gdn":
        def step(s):
            return sf.segmented_gdn_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], w.n_seg, scale=w.scale,
                                        output_final_state=True)
    elif w.name == "ssd_gla":
        def step(s):
            return sf.segmented_gla_fwd(s["q"], s["k"], s["v"], s["g"], w.n_seg, scale=w.scale, chunk=w.chunk,
                                        output_final_state=True)
    else:
        raise ValueError(w.name)
    return step


def cpu_baseline(w):
    """The oracle, as it stands, on the host cores: its float32 build of the token loops (the CPU
    throughput baseline; parity uses the float64 build) over one pass of the workload, or a bounded
    head sample of it."""
    import oracle
    import workloads as wl
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    threads = min(threads, len(os.sched_getaffinity(0)))
    model = cpu_model()
    f = wl.to_f32
    if isinstance(w, wl.GateWorkload):
        log("cpu_baseline: float64 gate-transform oracle (numpy) ...")
        t0 = time.perf_counter()
        oracle.gate_transform(f(w.raw), f(w.A_log), f(w.dt_bias), w.kind, w.lower_bound)
        dt = time.perf_counter() - t0
        return {"value": w.tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle", "precision": "f64",
                "cpu_model": model,
                "sample": f"the whole {w.name} workload ({w.raw.numel()} gates), one float64 pass, {dt:.2f} s wall"}
    if isinstance(w, wl.DecodeWorkload):
        log("cpu_baseline: float64 decode oracle (numpy, one step) ...")
        t0 = time.perf_counter()
        if w.per_channel:
            oracle.kda_decode(f(w.packed_qkv), f(w.raw_gate), f(w.raw_beta), f(w.A_log), f(w.dt_bias), f(w.pool),
                              w.state_indices.numpy(), None, H=w.H, K=w.K, V=w.V, kind=w.gate_kind,
                              lower_bound=w.lower_bound, scale=w.scale)
        else:
            oracle.gdn_decode(f(w.packed_qkv), f(w.raw_gate), f(w.raw_beta), f(w.A_log), f(w.dt_bias), f(w.pool),
                              w.state_indices.numpy(),
                              None if w.has_initial_state is None else w.has_initial_state.numpy(),
                              H=w.H, HK=w.HK, K=w.K, V=w.V, scale=w.scale)
        dt = time.perf_counter() - t0
        return {"value": w.tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle", "precision": "f64",
                "cpu_model": model,
                "sample": f"the whole {w.name} step ({w.tokens} rows x {w.H} heads), one float64 pass, "
                          f"{dt:.2f} s wall"}
    if w.name == "dense_gdn_bwd":
        log(f"cpu_baseline: float64 backward oracle on {threads} threads ...")
        t0 = time.perf_counter()
        oracle.gdn_backward(f(w.q), f(w.k), f(w.v), f(w.g), f(w.beta), f(w.meta["do"]), f(w.h0), f(w.meta["dht"]),
                            scale=w.scale, threads=threads)
        dt = time.perf_counter() - t0
        return {"value": w.tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "precision": "f64",
                "cpu_model": model,
                "sample": f"the whole {w.name} workload ({w.tokens} tokens x {w.H} heads), one float64 pass of the "
                          f"reverse-mode token loop, {dt:.2f} s wall"}
    if w.name == "dense_kda":
        log("cpu_baseline: float64 KDA oracle (numpy token loop) ...")
        t0 = time.perf_counter()
        oracle.kda_forward(f(w.q), f(w.k), f(w.v), f(w.g), f(w.beta), f(w.h0), scale=w.scale)
        dt = time.perf_counter() - t0
        return {"value": w.tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle", "precision": "f64",
                "cpu_model": model,
                "sample": f"the whole {w.name} workload ({w.tokens} tokens x {w.H} heads), one float64 pass of the "
                          f"numpy token loop, {dt:.2f} s wall"}
    if w.name in ("recurrent_kda", "recurrent_gdn", "paged_gdn"):
        args = dict(q=f(w.q), k=f(w.k), v=f(w.v), g=f(w.g))
        log(f"cpu_baseline: float64 oracle on {threads} threads ...")
        t0 = time.perf_counter()
        if w.name == "recurrent_kda":
            pool, idx = f(w.meta["pool"]), w.meta["state_indices"].numpy()
            oracle.kda_forward(args["q"], args["k"], args["v"], args["g"], f(w.beta), pool[idx], scale=w.scale)
        else:
            oracle.gdn_recurrent_paged(args["q"], args["k"], args["v"], args["g"], f(w.beta), f(w.meta["pool"]),
                                       w.meta["state_indices"].numpy(),
                                       cu_seqlens=None if w.cu_seqlens is None else w.cu_seqlens.numpy(),
                                       scale=w.scale)
        dt = time.perf_counter() - t0
        return {"value": w.tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "precision": "f64",
                "cpu_model": model,
                "sample": f"the whole {w.name} workload ({w.tokens} tokens x {w.H} heads), one float64 pass, "
                          f"{dt:.2f} s wall"}
    # Chunk workloads: the float32 token loops. Whole workload when it is small; otherwise a sample
    # of heads (each (sequence, head) chain costs the same per token, so tokens/s scales by H/heads)
    # sized to stay within about half a minute on the host.
    heads = w.H
    if w.tokens * w.H > 40_000_000:
        heads = max(w.H // w.HK, (w.H * 40_000_000) // (w.tokens * w.H) // (w.H // w.HK) * (w.H // w.HK))
    grp = w.H // w.HK
    hs = list(range(heads))
    gs = sorted({h // grp for h in hs})
    sub = lambda x, idx: x[:, :, idx]
    q, k = f(sub(w.q, gs)), f(sub(w.k, gs))
    v, g = f(sub(w.v, hs)), f(sub(w.g, hs))
    beta = None if w.beta is None else f(sub(w.beta, hs))
    h0 = None if w.h0 is None else f(w.h0[:, hs])
    cu = None if w.cu_seqlens is None else w.cu_seqlens.numpy()
    kind = "gdn" if w.kind == "gdn" else "gla"
    log(f"cpu_baseline: float32 oracle token loops on {threads} threads, {heads}/{w.H} heads ...")
    # whole passes until at least 3 s have run (one pass when a pass takes longer)
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.forward_f32(kind, q, k, v, g, beta, h0, cu_seqlens=cu, scale=w.scale, threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 3.0:
            break
    frac = heads / w.H
    return {"value": w.tokens * frac * passes / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "precision": "f32", "cpu_model": model,
            "sample": f"{w.name}: {'all' if heads == w.H else heads} of {w.H} heads over all {w.tokens} tokens, "
                      f"{passes} pass(es) of the float32 token loops, {dt:.2f} s wall; tokens/s scaled by heads/H"}


def measured_copy_gbs(dev, nbytes=1 << 30, reps=10):
    """HBM bandwidth a plain device-to-device copy reaches here (bytes read plus bytes written per
    second), for a buffer far larger than the caches: the practical ceiling next to the spec peak.
    Timed with events on torch's current stream, which is where the copy runs."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    return round(gbs, 1)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=3, help="input sets cycled through (cache defeat)")
    ap.add_argument("--workload", default="dense_gdn",
                    choices=["dense_gdn", "tiny_gdn", "varlen_gdn", "long_gdn", "ssd_gla", "decode_gdn",
                             "recurrent_gdn", "gate_transform", "paged_gdn", "recurrent_kda", "decode_kda",
                             "dense_gdn_bwd", "dense_kda"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true",
                    help="skip the second pass, whose launches are bracketed with HIP events")
    ap.add_argument("--no-copy-peak", action="store_true",
                    help="skip the measured-copy bandwidth reported beside the spec peak")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 512 MiB device-to-device copy three times (reference dispatches "
                         "that scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings to bytes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (one GPU's share of the "
              "work is what it runs); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunked_linear_recurrence_amd as sf
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    sf.lib()

    log(f"bench: generating {args.workload} ...")
    w = wl.CONFIGS[args.workload]()
    sets = make_sets(w, dev, max(1, args.rotate))
    step = step_fn(w)

    log(f"bench: warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # Pass 1: the timed steps as a caller runs them (value, ms_per_step). Pass 2: the same steps with
    # every launch bracketed by HIP events on its stream (per-kernel durations for the roofline);
    # the event records add small gaps between launches, so pass 2's wall time is reported apart.
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Pass 1b: the same steps with one event on torch's current stream (the launch stream) between
    # consecutive steps: per-step durations for p50 and min.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        step(sets[i % len(sets)])
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    p50_ms = per_step[len(per_step) // 2] if len(per_step) % 2 else 0.5 * (per_step[len(per_step) // 2 - 1] +
                                                                          per_step[len(per_step) // 2])
    min_ms = per_step[0]
    kt, ev_elapsed = {}, None
    if not args.no_events:
        log(f"bench: timing {args.steps} steps with per-launch events")
        sf.timing_enable(64 * (args.steps + 1))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            step(sets[i % len(sets)])
        torch.cuda.synchronize()
        ev_elapsed = time.perf_counter() - t1
        kt = sf.timing_collect()
        sf.timing_enable(0)

    ms_per_step = 1e3 * elapsed / args.steps
    value = w.tokens * args.steps / elapsed
    kernels = {k: {"launches": n, "avg_us": 1e3 * ms / n} for k, (n, ms) in kt.items()}
    log("bench: per-kernel " + json.dumps(kernels))

    roof = None
    if kernels:
        dom = max(kt, key=lambda k: kt[k][1])
        avg_s = kt[dom][1] / kt[dom][0] / 1e3
        ab = algorithmic_bytes(w, dom)
        ach = ab / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic_from_profile(dom, w.name),
                "kernel": dom, "avg_us": round(avg_s * 1e6, 2), "algorithmic_bytes": ab}
        if dom == "gdn_bwd_grad":
            # the gradient kernel's contractions take operands of the input type (float32 or bf16 MFMA): its
            # roofline is whichever floor is higher, the contractions' at that type's peak or the HBM bytes',
            # and the other one is reported beside it
            fl = bwd_grad_flops(w)
            tf = fl / avg_s / 1e12
            bf = w.q.dtype == torch.bfloat16
            peak = BF16_PEAK_TFLOPS if bf else F32_PEAK_TFLOPS
            mf = {"bound": "mfma", "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                  "frac": round(tf / peak, 4), "traffic": roof["traffic"], "kernel": dom, "avg_us": roof["avg_us"],
                  "algorithmic_flops": fl, "dtype": "bf16" if bf else "f32"}
            if fl / (peak * 1e12) > ab / (HBM_PEAK_GBS * 1e9):
                mf["hbm"] = roof
                roof = mf
            else:
                roof["mfma"] = mf
    decode = isinstance(w, wl.DecodeWorkload)
    gate = isinstance(w, wl.GateWorkload)
    path_bytes = algorithmic_bytes(w, "decode_path" if decode else "gate_path" if gate else "path")
    path_ach = path_bytes / (elapsed / args.steps) / 1e9
    copy_gbs = None if args.no_copy_peak else measured_copy_gbs(dev)
    if roof is not None and copy_gbs and roof["bound"] == "hbm":
        roof["measured_peak"] = copy_gbs
        roof["frac_of_measured"] = round(roof["achieved"] / copy_gbs, 4)

    out = {
        "metric": {"dense_gdn_bwd": METRIC_BWD, "dense_kda": METRIC_KDA}.get(w.name, METRIC), "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "p50_ms": p50_ms, "min_ms": min_ms,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if (w.packed_qkv if decode else w.raw if gate else w.q).dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": ({"workload": w.name, "shape": list(w.raw.shape), "kind": w.kind, "tokens": w.tokens,
                    "rotate": len(sets)} if gate else
                   {"workload": w.name, "B": w.B, "H": w.H, "HK": w.HK, "K": w.K, "V": w.V,
                    "pool": "f32" if w.pool.dtype == torch.float32 else "bf16", "num_slots": w.pool.shape[0],
                    "tokens": w.tokens, "rotate": len(sets)} if decode else
                   {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "HK": w.HK, "K": w.K, "V": w.V,
                    "chunk": w.chunk, "n_seg": w.n_seg, "tokens": w.tokens, "rotate": len(sets)}),
        "roofline": roof,
        "path_roofline": {"bound": "hbm", "achieved": round(path_ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(path_ach / HBM_PEAK_GBS, 4), "algorithmic_bytes": path_bytes,
                          "measured_peak": copy_gbs,
                          "frac_of_measured": None if not copy_gbs else round(path_ach / copy_gbs, 4)},
        "path_roofline_two_pass": None,
        "kernels": kernels,
        "events_pass_ms_per_step": None if ev_elapsed is None else 1e3 * ev_elapsed / args.steps,
        "cpu_baseline": None,
    }
    tp = None if (decode or gate) else two_pass_bytes(w)
    if tp:
        tp_ach = tp / (elapsed / args.steps) / 1e9
        out["path_roofline_two_pass"] = {"bound": "hbm", "achieved": round(tp_ach, 1), "peak": HBM_PEAK_GBS,
                                         "unit": "GB/s", "frac": round(tp_ach / HBM_PEAK_GBS, 4),
                                         "algorithmic_bytes": tp}
    if args.copy_calibration:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = {"read": n, "write": n}
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

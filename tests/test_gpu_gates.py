"""GPU parity of the gate transform (sf_gate_transform through the C ABI) against the float64 oracle
(oracle.gate_transform, pinned in tests/test_oracle_decode.py). The arithmetic is float32 on both
sides of the float64 reference: max |x - oracle| <= 1e-4 max(1, |oracle|) for every element."""
import sys

import numpy as np
import pytest
import torch

import chunked_linear_recurrence_amd as sf
import oracle
import workloads as wl

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sf.lib()
    return torch.device("cuda:0")


CASES = [
    # name, shape, H, D (None = per-head), dtype, kind, lower bound
    ("head-bf16-softplus", (2, 300, 16), 16, None, torch.bfloat16, "softplus", None),
    ("head-f32-bounded", (1, 77, 6), 6, None, torch.float32, "bounded", -5.0),
    ("head-tail", (7, 3), 3, None, torch.float32, "softplus", None),       # 21 gates: a ragged last vector
    ("channel-bf16-bounded", (2, 64, 4, 128), 4, 128, torch.bfloat16, "bounded", -5.0),
    ("channel-f32-softplus", (3, 33, 2, 64), 2, 64, torch.float32, "softplus", None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gate_transform_vs_oracle(dev, case):
    name, shape, H, D, dt, kind, lb = case
    say(f"gate transform {name}: {shape}")
    d = wl.gate_inputs(shape=shape, H=H, D=D, dtype=dt, seed=len(name))
    d["raw"] = d["raw"] * 3.0  # reach both tails of softplus and sigmoid
    out = sf.gate_transform(d["raw"].to(dev), d["A_log"].to(dev), d["dt_bias"].to(dev), kind=kind, lower_bound=lb)
    torch.cuda.synchronize()
    ref = oracle.gate_transform(wl.to_f32(d["raw"]), wl.to_f32(d["A_log"]), wl.to_f32(d["dt_bias"]), kind, lb)
    got = out.cpu().numpy()
    assert got.shape == ref.shape and got.dtype == np.float32
    err = float(np.max(np.abs(got - ref) / np.maximum(1.0, np.abs(ref))))
    say(f"{name}: max scaled err {err:.3g}")
    assert err <= 1e-4
    assert np.all(got <= 0) and (lb is None or np.all(got >= lb))


def test_gate_transform_full_size(dev):
    w = wl.gate_transform()
    say("gate transform: full-size workload")
    out = sf.gate_transform(w.raw.to(dev), w.A_log.to(dev), w.dt_bias.to(dev), kind=w.kind)
    torch.cuda.synchronize()
    ref = oracle.gate_transform(wl.to_f32(w.raw), wl.to_f32(w.A_log), wl.to_f32(w.dt_bias), w.kind)
    err = float(np.max(np.abs(out.cpu().numpy() - ref) / np.maximum(1.0, np.abs(ref))))
    say(f"gate_transform: max scaled err {err:.3g}")
    assert err <= 1e-4

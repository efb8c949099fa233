"""Helpers for the GPU parity tests: generate inputs on the GPU, hand the same
bytes to the HIP library and (as numpy) to the oracle, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

from fixtures import moe_inputs as fx
from oracle import moe_oracle as ora

# Output tolerance of the layer (FP16 outputs vs the float64 oracle).
REL_L2_TOL = 2e-3
MAX_ABS_TOL = 5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got, want) -> float:
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    return float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-300))


def max_abs(got, want) -> float:
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - np.asarray(want, dtype=np.float64))))


def assert_close(got, want, what=""):
    r, m = rel_l2(got, want), max_abs(got, want)
    say(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= REL_L2_TOL and m <= MAX_ABS_TOL, (what, r, m)
    return r, m


def gpu_layer(shape, cfg, layer):
    """Weights generated on the GPU; returns the numpy copy both sides use."""
    w = fx.layer_weights(shape, cfg, layer, device="cuda")
    return {k: v.cpu().numpy() for k, v in w.items()}


def to_gpu(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


def flip_is_explained(x_gpu, x_ora, router, ids_gpu, ids_ora):
    """True when every expert that differs between the two selections is
    within the logit change that the difference of the two inputs can cause:
    for a chosen by the oracle only and b by the GPU only,
    logit_ora(a) - logit_ora(b) <= B_a + B_b with B_e = sum_i |dx_i| |Wr_ei|
    (logits on the oracle's input, exact)."""
    dx = np.abs(x_gpu.astype(np.float64) - x_ora.astype(np.float64))
    B = np.abs(router.astype(np.float64)) @ dx
    lg = ora.router_logits(x_ora[None, :], router)[0].astype(np.float64)
    only_o = sorted(set(ids_ora.tolist()) - set(ids_gpu.tolist()))
    only_g = sorted(set(ids_gpu.tolist()) - set(ids_ora.tolist()))
    worst = max((lg[a] - lg[b]) - (B[a] + B[b]) for a in only_o for b in only_g) if only_o else -1.0
    return worst <= 0.0, worst

"""Helpers for the GPU parity tests: generate inputs on the GPU, hand the same
bytes to the HIP library and (as numpy) to the oracle, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

from fixtures import moe_inputs as fx

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

"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and compare."""
from __future__ import annotations

import sys

import numpy as np

import oracle

TOL_F32 = 1e-5  # float32 inputs, float32 state and outputs
TOL_BF16 = 2e-3  # bfloat16 inputs, float32 state and outputs


def say(*msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu-case]", *msg, file=sys.stderr, flush=True)


def to_dev(x: dict, device="cuda"):
    import torch

    out = {}
    for n in "rwkvab":
        a = x[n]
        if a.dtype == np.uint16:
            out[n] = torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            out[n] = torch.from_numpy(a).to(device)
    s = x.get("state_in")
    out["state_in"] = None if s is None else torch.from_numpy(s).to(device)
    return out


def rel(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    d = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return d / m if m > 0 else d


def oracle_units(x: dict, units):
    """Oracle on selected (b, h) units only. Returns {(b,h): (y [T,N], state [N,N])}."""
    res = {}
    for (b, h) in units:
        sl = {n: np.ascontiguousarray(x[n][b:b + 1, :, h:h + 1, :]) for n in "rwkvab"}
        s = x.get("state_in")
        s_in = None if s is None else np.ascontiguousarray(s[b:b + 1, h:h + 1])
        y, st = oracle.wkv7(*(sl[n] for n in "rwkvab"), state_in=s_in)
        res[(b, h)] = (y[0, :, 0, :], st[0, 0])
    return res


def sample_units(B, H, n, seed=0):
    rng = np.random.default_rng(seed)
    units = {(0, 0), (B - 1, H - 1)}
    while len(units) < min(n, B * H):
        units.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(units)

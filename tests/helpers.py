"""Shared test utilities: tolerances, device/host transfers, lazily fetched expert weights."""
from __future__ import annotations

import re
import os

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Tolerances of the parity bar: bf16 paths (fp32 accumulation) max|err| <= 2e-2 * max|ref|; fp32
# paths max|err| <= 1e-4 * max|ref|.
TOL = {"bf16": 2e-2, "f32": 1e-4}
NEAR_TIE = 1e-4  # tokens whose k-th and (k+1)-th logits differ by less are excluded end to end


def dkey(dtype) -> str:
    return "f32" if dtype in (torch.float32, "f32") else "bf16"


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def max_rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err / scale if scale > 0 else err


def assert_parity(got, ref, dtype, what=""):
    r = max_rel_err(got, ref)
    tol = TOL[dkey(dtype)]
    assert r <= tol, f"{what}: max|err|/max|ref| = {r:.3e} > {tol:.0e}"
    return r


class ExpertSlices:
    """W[e] -> expert e's weight matrix as float64 numpy, copied from the device on demand and
    cached (the oracle indexes weights by expert only)."""

    def __init__(self, t: torch.Tensor, cache: bool = True):
        self.t = t
        self.cache = {} if cache else None

    def __getitem__(self, e):
        e = int(e)
        if self.cache is None:
            return to_np(self.t[e]).astype(np.float64)
        if e not in self.cache:
            self.cache[e] = to_np(self.t[e]).astype(np.float64)
        return self.cache[e]

    def __len__(self):
        return self.t.shape[0]


def oracle_weights(W: dict, cache: bool = True) -> dict:
    """Device weights -> what the oracle takes: small tensors as float64 numpy, expert stacks lazily."""
    out = {"W_R": to_np(W["W_R"]).astype(np.float64),
           "bias": None if W.get("bias") is None else to_np(W["bias"]).astype(np.float64),
           "W1": ExpertSlices(W["W1"], cache), "W2": ExpertSlices(W["W2"], cache),
           "W3": ExpertSlices(W["W3"], cache)}
    for key in ("Ws1", "Ws2", "Ws3"):
        out[key] = None if W.get(key) is None else to_np(W[key]).astype(np.float64)
    return out


def header_exports() -> list:
    """Function names declared in include/*.h."""
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if not f.endswith(".h"):
            continue
        src = open(os.path.join(inc, f)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, re.M):
            names.append(m.group(1))
    return sorted(set(names))

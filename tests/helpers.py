"""Shared test utilities: tolerances, device/host transfers, lazily fetched expert weights."""
from __future__ import annotations

import re
import os

import numpy as np
import torch

import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Tolerances of the parity bar: bf16 paths (fp32 accumulation) max|err| <= 2e-2 * max|ref|; fp32
# paths max|err| <= 1e-4 * max|ref|.
TOL = {"bf16": 2e-2, "f32": 1e-4}
NEAR_TIE = 1e-4  # tokens whose k-th and (k+1)-th logits differ by less are excluded end to end

# The tighter bar, against the oracle run with the implementation's storage rounding mirrored
# (`store`: the expert hidden H and the outputs Y, S rounded to bf16).  With the same values stored,
# the two sides differ only where fp32 accumulation (GPU) and fp64 accumulation (oracle) land on
# opposite sides of a bf16 rounding midpoint: a stored output then differs by one bf16 unit, and a
# hidden value that flipped moves the next product by a small multiple of the output's rms.  Bar for
# a bf16-stored output:  |got - ref| <= ulp_bf16(ref) + MIRROR_BETA * rms(ref), element by element.
# A CPU emulation of the kernels' arithmetic (fp32 sums per 32-wide K step, bf16 H and Y) at the
# DeepSeek-V3 and V2-Lite expert shapes uses at most 0.74 of it; a 1% error on a tile fails it.
MIRROR_BETA = 2.0 ** -8

# The backward pass's FarSkip stack test (tests/test_gpu_backward.py): its shapes, its modes and
# masks, and the top-k margin its inputs keep at every layer.  Each side runs its own forward, so the
# layer inputs drift apart by bf16 rounding flips; tests/test_tie_margin_cpu.py measures that drift
# (kernel arithmetic emulated against the store-mirrored oracle, these shapes and cases): the logits
# move by at most 1.1e-2 by the third layer, so two logits closer than 2.2e-2 may swap order; the
# margin is 0.05, more than twice that.
BWD_STACK = {"T": 256, "d": 128, "E": 8, "k": 2, "c": 128, "cs": 128, "L": 3, "gate": "softmax", "renorm": True}
BWD_STACK_CASES = [("none", None), ("partial", None), ("outdated", None), ("partial", [1, 0, 1]),
                   ("outdated", [0, 1, 1])]
BWD_TIE_MARGIN = 0.05


def make_layer(seed, T, d, E, c, cs, bias, empty=()):
    """Seeded bf16 input A, weights W and output gradient dOut of one sublayer for the backward
    tests (weights N(0, 1/fan_in); a router bias N(0, 0.5^2) when asked, -1e4 for `empty` experts)."""
    g = lambda i, shape, std: mi.normal(shape, std, mi.seed_for(89, seed, i), "cpu", torch.bfloat16)
    W = {"W_R": g(1, (E, d), d ** -0.5), "W1": g(2, (E, c, d), d ** -0.5), "W2": g(3, (E, c, d), d ** -0.5),
         "W3": g(4, (E, d, c), c ** -0.5)}
    W["bias"] = mi.normal((E,), 0.5, mi.seed_for(89, seed, 5)) if bias else None
    if W["bias"] is not None:
        for e in empty:
            W["bias"][e] = -1e4
    if cs:
        W["Ws1"], W["Ws2"] = g(6, (cs, d), d ** -0.5), g(7, (cs, d), d ** -0.5)
        W["Ws3"] = g(8, (d, cs), cs ** -0.5)
    A = g(9, (T, d), 1.0)
    dOut = mi.normal((T, d), 1.0, mi.seed_for(89, seed, 10))
    return A, W, dOut


# achieved errors of every float comparison, printed at the end of the session (conftest.py)
RESULTS = []


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


def _current_test() -> str:
    return os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0].split("::")[-1]


def report(what: str, **vals) -> None:
    """Record an achieved error (printed in the session summary) and print it at once."""
    RESULTS.append((_current_test(), what, vals))
    print(f"[parity] {_current_test()} {what}: " + ", ".join(f"{k}={v:.3e}" for k, v in vals.items()), flush=True)


def assert_parity(got, ref, dtype, what=""):
    r = max_rel_err(got, ref)
    tol = TOL[dkey(dtype)]
    report(what, rel=r, bar=tol)
    assert r <= tol, f"{what}: max|err|/max|ref| = {r:.3e} > {tol:.0e}"
    return r


def bf16_ulp(x) -> np.ndarray:
    """Spacing of the bfloat16 values around |x|: 2^(e-7) for 2^e <= |x| < 2^(e+1) (8 significant
    bits); values below the smallest normal take the smallest normal's spacing."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def rms(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 0.0


def mirror_bound(ref) -> np.ndarray:
    """Element-wise bar of a bf16-stored output against the store-mirrored oracle."""
    ref = np.asarray(ref, dtype=np.float64)
    return bf16_ulp(ref) + MIRROR_BETA * rms(ref)


def assert_mirror(got, ref, what="", bound=None) -> float:
    """|got - ref| <= bound element by element (default: mirror_bound(ref)); records and returns the
    largest |got - ref| / bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    bound = mirror_bound(ref) if bound is None else np.asarray(bound, dtype=np.float64)
    ratio = float(np.max(np.abs(got - ref) / bound))
    report(what + " (mirror)", rel=max_rel_err(got, ref), of_bar=ratio)
    assert ratio <= 1.0, f"{what}: |err| reaches {ratio:.3f} of the mirrored-oracle bar"
    return ratio


def combine_bound(S, Y, topk_w, dest_row, o_prev=None) -> np.ndarray:
    """Element-wise bar of a layer output S + sum_i w_i Y[dest_row[t, i]] formed in fp32 from the
    bf16-stored S and Y, against the store-mirrored oracle: each stored value within its own bar
    (mirror_bound over all of S, resp. all of Y), weighted as the combine weights it, plus one fp32
    rounding per addition (k + 2 of them, on magnitudes up to |o_prev| + |S| + sum_i w_i |Y_i|).
    S: [n, d] (zeros without shared experts); Y: [N, d] in grouped row order; topk_w, dest_row:
    [n, k] for the n compared tokens; o_prev: [n, d] residual added in the same sums, or None."""
    S = np.asarray(S, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    w = np.asarray(topk_w, dtype=np.float64)
    dest = np.asarray(dest_row, dtype=np.int64)
    k = w.shape[1]
    y_floor = MIRROR_BETA * rms(Y)
    bound = bf16_ulp(S) + MIRROR_BETA * rms(S) if np.any(S) else np.zeros_like(S)
    mag = np.abs(S) + (0.0 if o_prev is None else np.abs(np.asarray(o_prev, dtype=np.float64)))
    for i in range(k):
        Yi = Y[dest[:, i]]
        bound = bound + w[:, i:i + 1] * (bf16_ulp(Yi) + y_floor)
        mag = mag + w[:, i:i + 1] * np.abs(Yi)
    return bound + (k + 2) * 2.0 ** -24 * mag


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 copied as is and widened on the host, exactly)."""
    return t.detach().cpu().to(torch.float64).numpy()


class ExpertSlices:
    """W[e] -> expert e's weight matrix as float64 numpy, copied from the device on demand and
    cached (the oracle indexes weights by expert only)."""

    def __init__(self, t: torch.Tensor, cache: bool = True):
        self.t = t
        self.cache = {} if cache else None
        self.fetched = set()   # experts copied at least once

    def __getitem__(self, e):
        e = int(e)
        self.fetched.add(e)
        if self.cache is None:
            return to_f64(self.t[e])
        if e not in self.cache:
            self.cache[e] = to_f64(self.t[e])
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

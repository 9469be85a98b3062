"""Seeded synthetic inputs for the MoE sublayer and the FarSkip stack.

This module is shared by the HIP-path tests, the bench and the CPU oracle's callers. It holds the
workload shapes, the value distributions and seeded draws only: no router, no top-k, no MLP, no
permutation and no combine arithmetic lives here.

Workloads (shapes as the FarSkip-Collective pages name the models they convert and measure:
DeepSeek-V2-Lite, Qwen3-30B-A3B, Llama-4-Scout, DeepSeek-V3; the expert dimensions are the public
model shapes, the values are synthetic, no checkpoint is used):

  tiny-fp32          T=64     d=128  E=8   k=2  c=256   no shared      softmax, renormalised, fp32
  dsv2-lite          T=4096   d=2048 E=64  k=6  c=1408  2 x 1408 shared softmax, not renormalised
  qwen3-30b-a3b      T=8192   d=2048 E=128 k=8  c=768   no shared      softmax, renormalised,
                                                                        per-expert N(0,1) logit bias
  llama4-scout       T=8192   d=5120 E=16  k=1  c=8192  1 x 8192 shared sigmoid, not renormalised
  dsv3-stack         T=65536  d=7168 E=256 k=8  c=2048  1 x 2048 shared sigmoid, renormalised,
                                                                        4 FarSkip layers (partial)

Values: activations N(0,1); weights N(0, 0.02^2) (tiny-fp32: W_R, W1, W2 ~ N(0, 1/d), W3 ~ N(0, 1/c)).
Every tensor is drawn in fp32 from its own seed, derived from (20251101, config id, layer, tensor id,
expert), and rounded to bf16 (round to nearest even) where the workload is bf16.  Draws use torch's
generator on the device the tensor lives on, so one seed gives one tensor per device type; a test
draws once and copies to where it is needed.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

BASE_SEED = 20251101

# tensor ids used in the seed derivation
T_ACT, T_WR, T_BIAS, T_W1, T_W2, T_W3, T_WS1, T_WS2, T_WS3 = 0, 1, 2, 3, 4, 5, 6, 7, 8
T_LOGITS, T_TOPK, T_GROUPS, T_GATEW, T_PERM, T_Y, T_SAMPLE, T_MISC = 10, 11, 12, 13, 14, 15, 16, 17
T_WA1, T_WA2, T_WA3 = 18, 19, 20   # the dense block standing in for a layer's attention sub-block


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    cfg_id: int
    name: str
    T: int
    d: int
    E: int
    k: int
    c: int
    n_shared: int
    c_shared: int
    gate: str            # "softmax" | "sigmoid"
    renormalize: bool
    dtype: str           # "f32" | "bf16"
    layers: int = 1
    router_bias: bool = False
    w_std: float = 0.02  # W_R, W1, W2 (and shared W1, W2)
    w3_std: float = 0.02  # W3 (and shared W3)
    weight_cfg_id: Optional[int] = None  # draw the weights of that workload (same shapes) instead

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def shared_width(self) -> int:
        return self.n_shared * self.c_shared

    def scaled(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    def flops_per_token(self) -> dict:
        """Algorithmic FLOP per token: router, routed experts, shared experts (per layer)."""
        router = 2 * self.d * self.E
        routed = 6 * self.d * self.c * self.k
        shared = 6 * self.d * self.shared_width
        return {"router": router, "routed": routed, "shared": shared,
                "total": router + routed + shared}


CONFIGS = [
    MoEConfig(0, "tiny-fp32", T=64, d=128, E=8, k=2, c=256, n_shared=0, c_shared=0,
              gate="softmax", renormalize=True, dtype="f32",
              w_std=1.0 / 128 ** 0.5, w3_std=1.0 / 256 ** 0.5),
    MoEConfig(1, "dsv2-lite", T=4096, d=2048, E=64, k=6, c=1408, n_shared=2, c_shared=1408,
              gate="softmax", renormalize=False, dtype="bf16"),
    MoEConfig(2, "qwen3-30b-a3b", T=8192, d=2048, E=128, k=8, c=768, n_shared=0, c_shared=0,
              gate="softmax", renormalize=True, dtype="bf16", router_bias=True),
    MoEConfig(3, "llama4-scout", T=8192, d=5120, E=16, k=1, c=8192, n_shared=1, c_shared=8192,
              gate="sigmoid", renormalize=False, dtype="bf16"),
    MoEConfig(4, "dsv3-stack", T=65536, d=7168, E=256, k=8, c=2048, n_shared=1, c_shared=2048,
              gate="sigmoid", renormalize=True, dtype="bf16", layers=4),
    # one decode step of a 1024-sequence batch through the same 4 layers (same weights): every
    # expert gets about T*k/E = 32 rows, so the layer streams all of its weights for few tokens
    MoEConfig(5, "dsv3-decode", T=1024, d=7168, E=256, k=8, c=2048, n_shared=1, c_shared=2048,
              gate="sigmoid", renormalize=True, dtype="bf16", layers=4, weight_cfg_id=4),
]
BY_NAME = {c.name: c for c in CONFIGS}


def seed_for(cfg_id: int, layer: int, tensor: int, expert: int = 0, salt: int = 0) -> int:
    h = hashlib.blake2b(repr((BASE_SEED, cfg_id, layer, tensor, expert, salt)).encode(),
                        digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, seed: int, device="cpu", dtype=torch.float32) -> torch.Tensor:
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x if dtype == torch.float32 else x.to(dtype)


def block_scaled_normal(shape, std: float, seed: int, device="cpu", dtype=torch.bfloat16, spread: int = 4,
                        block: int = 32) -> torch.Tensor:
    """normal(shape, std) with each run of `block` consecutive elements along the last dimension
    multiplied by its own power of two 2^j, j uniform in [-spread, spread] (blocks whose magnitudes
    differ, as the rows of a block-scaled format see them)."""
    x = normal(shape, std, seed, device, torch.float32)
    nb = shape[-1] // block
    j = torch.randint(-spread, spread + 1, tuple(shape[:-1]) + (nb, 1), generator=_gen(seed + 1, device),
                      device=device)
    x = (x.view(*shape[:-1], nb, block) * torch.exp2(j.to(torch.float32))).view(shape)
    return x if dtype == torch.float32 else x.to(dtype)


def mx_random_codes(rows: int, cols: int, seed: int, device="cpu", scale_lo: int = 120, scale_hi: int = 134):
    """A random MXFP8 tensor: E4M3 codes uniform over the 254 finite codes [rows, cols] uint8 and
    E8M0 scale bytes uniform in [scale_lo, scale_hi] [rows, cols / 32] (inputs for a product whose
    operands are already quantised)."""
    g = _gen(seed, device)
    r = torch.randint(0, 254, (rows, cols), generator=g, device=device, dtype=torch.int32)
    codes = (r + (r >= 0x7F).to(torch.int32)).to(torch.uint8)      # skips the NaN codes 0x7F and 0xFF
    scales = torch.randint(scale_lo, scale_hi + 1, (rows, cols // 32), generator=g, device=device,
                           dtype=torch.int32).to(torch.uint8)
    return codes, scales


def mx_cancelling_codes(rows: int, cols: int, n_out: int, seed: int, device="cpu"):
    """MXFP8 operands (H [rows, cols], W [n_out, cols]) of a product H W^T whose 128-wide K chunks
    each hold one pair of large products that cancel exactly: in every chunk H is +v and -v at the
    chunk's first two columns (E4M3 exponent field 9 or 10, so |v| in [4, 16)) and W has one value
    there for both (field 6 to 8, positive); every other H element is small (field 1 or 2) with a
    random sign and every other W element is random (field 6 to 8, random sign).  All block scales
    are 2^0 (byte 127).  The exact result is then small beside the chunk's largest product, so a
    product's accumulation error is not hidden by the rounding of its output.
    Returns ((Hq, Hs), (Wq, Ws)) as uint8 tensors."""
    g = _gen(seed, "cpu")

    def field(lo, hi, shape):
        return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32)

    def code(sign, exp, man):
        return (sign << 7) | (exp << 3) | man

    Hq = code(field(0, 1, (rows, cols)), field(1, 2, (rows, cols)), field(0, 7, (rows, cols)))
    Wq = code(field(0, 1, (n_out, cols)), field(6, 8, (n_out, cols)), field(0, 7, (n_out, cols)))
    for k0 in range(0, cols, 128):
        big = code(torch.zeros((rows,), dtype=torch.int32), field(9, 10, (rows,)), field(0, 7, (rows,)))
        Hq[:, k0] = big
        Hq[:, k0 + 1] = big | 0x80
        w = code(torch.zeros((n_out,), dtype=torch.int32), field(6, 8, (n_out,)), field(0, 7, (n_out,)))
        Wq[:, k0] = w
        Wq[:, k0 + 1] = w
    Hs = torch.full((rows, cols // 32), 127, dtype=torch.uint8)
    Ws = torch.full((n_out, cols // 32), 127, dtype=torch.uint8)
    return ((Hq.to(torch.uint8).to(device), Hs.to(device)), (Wq.to(torch.uint8).to(device), Ws.to(device)))


def activations(cfg: MoEConfig, device="cpu", T: Optional[int] = None, layer: int = 0,
                dtype=None) -> torch.Tensor:
    """Token activations A (or the stack input o_0) [T, d] ~ N(0,1), in the workload dtype."""
    T = cfg.T if T is None else T
    return normal((T, cfg.d), 1.0, seed_for(cfg.cfg_id, layer, T_ACT, 0, T), device,
                  cfg.torch_dtype if dtype is None else dtype)


def weights_id(cfg: MoEConfig) -> int:
    """The workload id the weights are drawn for (a decode batch shares its prefill's weights)."""
    return cfg.cfg_id if cfg.weight_cfg_id is None else cfg.weight_cfg_id


def _stacked(cfg, layer, tensor, E, rows, cols, std, device, dtype):
    out = torch.empty((E, rows, cols), device=device, dtype=dtype)
    for e in range(E):
        out[e].copy_(normal((rows, cols), std, seed_for(weights_id(cfg), layer, tensor, e), device))
    return out


def layer_weights(cfg: MoEConfig, layer: int = 0, device="cpu") -> dict:
    """All weights of one MoE sublayer, in the layouts of the MLP equation (W1, W2: c x d; W3: d x c).

    Keys: W_R [E,d], bias [E] fp32 or None, W1 [E,c,d], W2 [E,c,d], W3 [E,d,c],
    Ws1 [ns*cs, d], Ws2 [ns*cs, d], Ws3 [d, ns*cs] (shared experts concatenated along the hidden
    dimension; shared expert s owns hidden rows/columns [s*cs, (s+1)*cs)), or None without shared.
    """
    dt = cfg.torch_dtype
    cid = weights_id(cfg)
    w = {}
    w["W_R"] = normal((cfg.E, cfg.d), cfg.w_std, seed_for(cid, layer, T_WR), device, dt)
    w["bias"] = (normal((cfg.E,), 1.0, seed_for(cid, layer, T_BIAS), device)
                 if cfg.router_bias else None)
    w["W1"] = _stacked(cfg, layer, T_W1, cfg.E, cfg.c, cfg.d, cfg.w_std, device, dt)
    w["W2"] = _stacked(cfg, layer, T_W2, cfg.E, cfg.c, cfg.d, cfg.w_std, device, dt)
    w["W3"] = _stacked(cfg, layer, T_W3, cfg.E, cfg.d, cfg.c, cfg.w3_std, device, dt)
    if cfg.n_shared:
        ns, cs = cfg.n_shared, cfg.c_shared
        w["Ws1"] = _stacked(cfg, layer, T_WS1, ns, cs, cfg.d, cfg.w_std, device, dt).reshape(ns * cs, cfg.d)
        w["Ws2"] = _stacked(cfg, layer, T_WS2, ns, cs, cfg.d, cfg.w_std, device, dt).reshape(ns * cs, cfg.d)
        ws3 = torch.empty((cfg.d, ns * cs), device=device, dtype=dt)
        for s in range(ns):
            ws3[:, s * cs:(s + 1) * cs].copy_(
                normal((cfg.d, cs), cfg.w3_std, seed_for(cid, layer, T_WS3, s), device))
        w["Ws3"] = ws3
    else:
        w["Ws1"] = w["Ws2"] = w["Ws3"] = None
    return w


def attn_weights(cfg: MoEConfig, layer: int, c_attn: int, device="cpu") -> dict:
    """Weights of the dense SwiGLU block that stands in for a layer's attention sub-block in the
    attention + MoE stack: Wa1, Wa2 [c_attn, d] ~ N(0, w_std^2), Wa3 [d, c_attn] ~ N(0, w3_std^2),
    in the workload dtype."""
    dt, cid = cfg.torch_dtype, weights_id(cfg)
    return {"Wa1": normal((c_attn, cfg.d), cfg.w_std, seed_for(cid, layer, T_WA1), device, dt),
            "Wa2": normal((c_attn, cfg.d), cfg.w_std, seed_for(cid, layer, T_WA2), device, dt),
            "Wa3": normal((cfg.d, c_attn), cfg.w3_std, seed_for(cid, layer, T_WA3), device, dt)}


def logits(T: int, E: int, seed: int, device="cpu", bias: Optional[torch.Tensor] = None,
           quantum: Optional[float] = None) -> torch.Tensor:
    """Synthetic fp32 router logits [T,E] ~ N(0,1) (+ per-expert bias).  With `quantum`, values are
    snapped to multiples of it so that many exact ties occur."""
    x = normal((T, E), 1.0, seed, device)
    if bias is not None:
        x = x + bias.to(device=device, dtype=torch.float32)[None, :]
    if quantum is not None:
        x = torch.round(x / quantum) * quantum
    return x.contiguous()


def topk_assignments(T: int, E: int, k: int, seed: int, device="cpu", zipf: float = 0.0) -> torch.Tensor:
    """Synthetic routing map [T,k] int32: k distinct experts per token, drawn without replacement,
    uniformly (zipf=0) or with Zipf-like expert popularity p_e ~ 1/(rank+1)^zipf over a seeded
    random ranking of the experts."""
    g = _gen(seed, "cpu")
    if zipf > 0:
        rank = torch.randperm(E, generator=g)
        p = 1.0 / (rank.to(torch.float64) + 1.0) ** zipf
    else:
        p = torch.ones(E, dtype=torch.float64)
    idx = torch.multinomial(p.expand(T, E).contiguous(), k, replacement=False, generator=g)
    return idx.to(torch.int32).to(device)


def group_sizes(n_rows: int, G: int, seed: int, zipf: float = 0.0, empty_groups=()) -> torch.Tensor:
    """Row counts per group [G] int64 summing to n_rows (multinomial, optional skew and forced-empty
    groups)."""
    g = _gen(seed, "cpu")
    p = torch.ones(G, dtype=torch.float64)
    if zipf > 0:
        rank = torch.randperm(G, generator=g)
        p = 1.0 / (rank.to(torch.float64) + 1.0) ** zipf
    for e in empty_groups:
        p[e] = 0.0
    if n_rows == 0:
        return torch.zeros(G, dtype=torch.int64)
    draws = torch.multinomial(p, n_rows, replacement=True, generator=g)
    return torch.bincount(draws, minlength=G)


def uniform(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    x = torch.rand(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x * (hi - lo) + lo


def randperm(n: int, seed: int, device="cpu") -> torch.Tensor:
    return torch.randperm(n, generator=_gen(seed, "cpu")).to(torch.int32).to(device)


def sample_rows(T: int, n: int, seed: int) -> torch.Tensor:
    """A seeded sorted subset of n distinct token rows out of T."""
    n = min(n, T)
    return torch.sort(torch.randperm(T, generator=_gen(seed, "cpu"))[:n]).values

"""Seeded synthetic MoE layers.

This module only draws inputs; it holds none of the layer's arithmetic.  Both
the GPU path's tests and the CPU oracle's tests take their inputs from here.

Workloads are routed MoE layers of a fine-grained MoE at inference ("Paper of
the Week #3 - Half the FLOPs Is Not Half the Time", section "The Receipt":
decode at batch 1 and 8, prefill), with experts made of 768-channel gated MLPs
("Channel Selection for Mixture-of-Experts Decoding Needs No Calibration Data",
section 2 "Background").  Trained weights are not available, so every tensor
is Gaussian:

* x ~ N(0, 1); for the bf16 layers each token is then RMS-normalised
  (x / sqrt(mean(x^2) + 1e-6)), as the input of an MoE block is;
* router weight Wr ~ N(0, var) with var = 1/H for the fp32 layer (logit std
  about 1) and var = 4/H for the bf16 layers (logit std about 2);
* optional router bias br ~ N(0, 0.5^2) for the skewed prefill workload;
* gate, up and down weights ~ N(0, 0.02^2), rounded to bf16 (RNE) for the
  bf16 layers.

A shared expert (``make_shared``: always run beside the routed experts, "Channel
Selection ..." appendix B) has Is channels drawn like an expert's, Sg and Su
[Is,H], Sd [H,Is], and an optional gate vector sg ~ N(0, 1/H) [H] fp32.

Seeds: each tensor has its own generator seeded with
``base + 1000 * layer + tensor_id`` (x=0, Wr=1, br=2, Wg=3, Wu=4, Wd=5, Sg=6,
Su=7, Sd=8, sg=9), so a layer is a pure function of (config, layer, base,
device).  The CPU and GPU
generators of torch draw different streams: a config's device is part of its
definition.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import torch

TENSOR_ID = {"x": 0, "Wr": 1, "br": 2, "Wg": 3, "Wu": 4, "Wd": 5, "Sg": 6, "Su": 7, "Sd": 8,
             "sg": 9}


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    I: int
    dtype: str  # "f32" or "bf16": activations and expert weights
    rms_norm_x: bool
    router_var_times_H: float  # Wr variance * H
    bias_std: float  # 0 = no router bias
    w_std: float = 0.02
    k_pairs: tuple = field(default_factory=tuple)
    layers: int = 1
    gen_device: str = "cpu"

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_T(self, T: int) -> "LayerConfig":
        return replace(self, T=T)


# The five workloads, smallest first.
TINY = LayerConfig("T8-H256-E16-I64-f32", T=8, H=256, E=16, I=64, dtype="f32",
                   rms_norm_x=False, router_var_times_H=1.0, bias_std=0.0,
                   k_pairs=((2, 4), (2, 2), (2, 16)))
_A3B_PAIRS = ((8, 8), (4, 4), (4, 16), (3, 16), (2, 16), (4, 128))
DECODE_B1 = LayerConfig("T1-H2048-E128-I768-bf16", T=1, H=2048, E=128, I=768,
                        dtype="bf16", rms_norm_x=True, router_var_times_H=4.0,
                        bias_std=0.0, k_pairs=_A3B_PAIRS)
DECODE_B8 = replace(DECODE_B1, name="T8-H2048-E128-I768-bf16", T=8)
PREFILL = LayerConfig("T4096-H2048-E128-I768-bf16-bias", T=4096, H=2048, E=128,
                      I=768, dtype="bf16", rms_norm_x=True,
                      router_var_times_H=4.0, bias_std=0.5,
                      k_pairs=((4, 16), (8, 8)))
LARGE = LayerConfig("L8-H4096-E512-I1024-bf16", T=1, H=4096, E=512, I=1024,
                    dtype="bf16", rms_norm_x=True, router_var_times_H=4.0,
                    bias_std=0.0, k_pairs=((10, 10), (5, 5), (5, 20)),
                    layers=8, gen_device="cuda")

CONFIGS = {c.name: c for c in (TINY, DECODE_B1, DECODE_B8, PREFILL, LARGE)}


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, seed, device):
    """N(0, std^2) fp32, drawn from its own seeded generator."""
    g = _gen(seed, device)
    return torch.randn(shape, generator=g, device=device,
                       dtype=torch.float32).mul_(std)


def _normal_cast(shape, std, seed, device, dtype):
    """Draw N(0, std^2) in fp32 and round to ``dtype`` (RNE).  Large tensors
    are drawn slice by slice along dim 0 from one generator, so peak memory
    stays near one fp32 slice; the slicing is fixed, so the draw is too."""
    if dtype == torch.float32:
        return _normal(shape, std, seed, device)
    g = _gen(seed, device)
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    per_row = 1
    for s in shape[1:]:
        per_row *= s
    step = max(1, (1 << 26) // max(per_row, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        tmp = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                          device=device, dtype=torch.float32)
        out[r0:r1] = tmp.mul_(std).to(dtype)
        del tmp
    return out


def make_x(cfg: LayerConfig, layer: int = 0, base: int = 0, device=None,
           T: int | None = None):
    device = device or cfg.gen_device
    T = cfg.T if T is None else T
    seed = base + 1000 * layer + TENSOR_ID["x"]
    x = _normal((T, cfg.H), 1.0, seed, device)
    if cfg.rms_norm_x:
        x = x / torch.sqrt(x.pow(2).mean(dim=1, keepdim=True) + 1e-6)
    return x.to(cfg.torch_dtype)


def make_weights(cfg: LayerConfig, layer: int = 0, base: int = 0, device=None):
    """Router and expert weights of one layer: dict Wr, br (or None), Wg, Wu, Wd.

    Layouts: Wr [E,H] fp32; br [E] fp32; Wg and Wu [E,I,H]; Wd [E,H,I]."""
    device = device or cfg.gen_device
    s = base + 1000 * layer
    H, E, I = cfg.H, cfg.E, cfg.I
    Wr = _normal((E, H), (cfg.router_var_times_H / H) ** 0.5,
                 s + TENSOR_ID["Wr"], device)
    br = None
    if cfg.bias_std > 0:
        br = _normal((E,), cfg.bias_std, s + TENSOR_ID["br"], device)
    wd = cfg.torch_dtype
    Wg = _normal_cast((E, I, H), cfg.w_std, s + TENSOR_ID["Wg"], device, wd)
    Wu = _normal_cast((E, I, H), cfg.w_std, s + TENSOR_ID["Wu"], device, wd)
    Wd = _normal_cast((E, H, I), cfg.w_std, s + TENSOR_ID["Wd"], device, wd)
    return {"Wr": Wr, "br": br, "Wg": Wg, "Wu": Wu, "Wd": Wd}


def make_shared(cfg: LayerConfig, Is: int, gate: bool = True, layer: int = 0, base: int = 0,
                device=None):
    """A shared expert of Is channels for the layer: dict Sg, Su [Is,H], Sd [H,Is]
    in the layer's dtype, and sg [H] fp32 (None without a gate)."""
    device = device or cfg.gen_device
    s = base + 1000 * layer
    wd = cfg.torch_dtype
    H = cfg.H
    out = {"Sg": _normal_cast((Is, H), cfg.w_std, s + TENSOR_ID["Sg"], device, wd),
           "Su": _normal_cast((Is, H), cfg.w_std, s + TENSOR_ID["Su"], device, wd),
           "Sd": _normal_cast((H, Is), cfg.w_std, s + TENSOR_ID["Sd"], device, wd),
           "sg": None}
    if gate:
        out["sg"] = _normal((H,), H ** -0.5, s + TENSOR_ID["sg"], device)
    return out


def make_layer(cfg: LayerConfig, layer: int = 0, base: int = 0, device=None,
               T: int | None = None):
    d = make_weights(cfg, layer, base, device)
    d["x"] = make_x(cfg, layer, base, device, T)
    return d


def to_numpy(t):
    """Host numpy view for the oracle: fp32 as float32, bf16 as uint16 bits."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()

"""Seeded synthetic workloads for the frame-wise GDN forward recurrence.

This module only draws random numbers and fixes shapes: it holds none of the
method's arithmetic, so both the oracle side and the HIP side of every test
can take their inputs from it.

Shapes follow the SANA-WM pages: a 60 s 720p clip is 961 latent frames
("NVIDIA Apresenta SANA-WM ...", section "1. Atencao Linear Hibrida com Gated
DeltaNet (GDN)"); a frame holds S spatial tokens of a latent grid (22 x 40 =
880 for 720p-shaped inputs, 45 x 80 = 3600 for the stress shape) and each head
carries a D x D state.  No dataset is used: Q, K, V are Gaussian, gamma and
beta uniform, drawn per (tensor, head) so that any single head can be
regenerated on its own.

Draw recipe (fixed; changing it changes every stored expectation):
  * one torch.Generator per (tensor, head), seeded with
      seed * 1_000_003 + stream_id,
    stream_id = tensor_index * B*H + b*H + h, tensor_index Q=0 K=1 V=2 gamma=3 beta=4;
  * Q, K, V: fp32 ``randn`` of shape [T, S, D] times the tensor's std, then
    rounded to nearest-even bf16, or to the nearest OCP E4M3 value (ties to
    even), when the I/O dtype is bf16 or fp8;
  * gamma, beta: fp32 ``rand`` of shape [T], mapped affinely onto [lo, hi].
CPU and GPU generators give different streams: a test draws on one device and
hands the same values to both sides.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional, Tuple

import torch

TENSORS = ("q", "k", "v", "gamma", "beta")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    S: int
    D: int
    dtype: str = "bf16"                 # I/O dtype of q, k, v, o: "bf16", "f32" or "fp8" (OCP E4M3)
    gamma: Tuple[float, float] = (0.9, 1.0)
    beta: Tuple[float, float] = (0.0, 1.0)
    q_std: float = 1.0
    k_std: float = 1.0
    v_std: float = 1.0
    beta_mode: str = "erase"
    chunk: int = 0                      # >0: frames per gdn_frame_step call

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.T * self.S

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.float8_e4m3fn}[self.dtype]

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the benchmark suite.
TINY = Workload("tiny-fp32 B1 H2 T8 S16 D16", 1, 2, 8, 16, 16, dtype="f32",
                gamma=(0.8, 1.0), beta=(0.0, 1.0))
SHORT = Workload("short-clip B1 H16 T81 S880 D64", 1, 16, 81, 880, 64,
                 gamma=(0.9, 1.0), beta=(0.2, 1.0))
MINUTE_720P = Workload("minute-720p B1 H20 T961 S880 D112", 1, 20, 961, 880, 112,
                       gamma=(0.95, 1.0), beta=(0.1, 1.0))
CHUNKED = SHORT.with_(name="chunked-rollout B1 H16 T81 S880 D64 chunk4", chunk=4)
STRESS = Workload("stress B2 H20 T961 S3600 D128", 2, 20, 961, 3600, 128,
                  gamma=(0.5, 1.0), beta=(1.0, 1.0), k_std=2.0)

ALL = (TINY, SHORT, MINUTE_720P, CHUNKED, STRESS)


def _gen(device, seed: int, stream_id: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + stream_id)
    return g


def head_tensors(w: Workload, b: int, h: int, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Inputs of one head: q, k, v [T, S, D] (I/O dtype), gamma, beta [T] fp32."""
    BH = w.B * w.H
    sid = lambda ti: ti * BH + b * w.H + h
    out = {}
    for ti, (name, std) in enumerate((("q", w.q_std), ("k", w.k_std), ("v", w.v_std))):
        x = torch.randn((w.T, w.S, w.D), generator=_gen(device, seed, sid(ti)),
                        device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[name] = x.to(w.torch_dtype)
    for ti, name, (lo, hi) in ((3, "gamma", w.gamma), (4, "beta", w.beta)):
        u = torch.rand((w.T,), generator=_gen(device, seed, sid(ti)), device=device,
                       dtype=torch.float32)
        out[name] = (u * (hi - lo) + lo) if hi != lo else torch.full_like(u, lo)
    return out


def generate(w: Workload, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """All heads: q, k, v [B, H, T, S, D]; gamma, beta [B, H, T] (fp32)."""
    q = torch.empty((w.B, w.H, w.T, w.S, w.D), dtype=w.torch_dtype, device=device)
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    gamma = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=device)
    beta = torch.empty_like(gamma)
    for b in range(w.B):
        for h in range(w.H):
            t = head_tensors(w, b, h, device, seed)
            q[b, h], k[b, h], v[b, h] = t["q"], t["k"], t["v"]
            gamma[b, h], beta[b, h] = t["gamma"], t["beta"]
    return {"q": q, "k": k, "v": v, "gamma": gamma, "beta": beta}


def to_numpy_io(x: torch.Tensor):
    """Host copy in the oracle's input convention: float32, uint16 bf16 bits or
    uint8 E4M3 codes."""
    x = x.detach().to("cpu").contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view("uint16")
    if x.dtype == torch.float8_e4m3fn:
        return x.view(torch.uint8).numpy()
    return x.numpy()


# ---------------------------------------------------------------------------
# Block-causal temporal convolution (the causal FFN of the SANA-Video talk).
#
# x [B, T, S, C] is one frame-major activation tensor: T latent frames of S
# spatial tokens with C channels.  No FFN width is given on the pages; the
# 720p-shaped workload takes C = 2240, the width 20 heads of D = 112 make, and
# the streaming chunk of 4 frames.  Draw recipe: x and the carried cache are
# fp32 ``randn`` rounded to the I/O dtype; the three taps w [3, C] and the bias
# [C] are fp32 ``rand`` mapped onto +-1/sqrt(3) (the default initialisation of
# a depthwise convolution with three taps); one generator per tensor, seeded
# seed * 1_000_003 + 7_000_000 + tensor index (x 0, w 1, bias 2, cache 3).

@dataclasses.dataclass(frozen=True)
class TconvWorkload:
    name: str
    B: int
    T: int
    S: int
    C: int
    chunk: int                          # frames per block of the chunk-causal generator
    dtype: str = "bf16"                 # I/O dtype of x, y and the cache: "bf16" or "f32"

    @property
    def tokens(self) -> int:
        return self.B * self.T * self.S

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]

    def with_(self, **kw) -> "TconvWorkload":
        return dataclasses.replace(self, **kw)


TCONV_720P = TconvWorkload("tconv-720p B1 T961 S880 C2240 chunk4", 1, 961, 880, 2240, 4)
TCONV_SMALL = TconvWorkload("tconv-small B2 T13 S40 C64 chunk4", 2, 13, 40, 64, 4)


def generate_tconv(w: TconvWorkload, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """x [B, T, S, C] and cache [B, S, C] in the I/O dtype; w [3, C] and bias [C] fp32."""
    base = seed * 1_000_003 + 7_000_000
    x = torch.randn((w.B, w.T, w.S, w.C), generator=_gen(device, base, 0), device=device,
                    dtype=torch.float32).to(w.torch_dtype)
    bound = 3.0 ** -0.5
    taps = torch.rand((3, w.C), generator=_gen(device, base, 1), device=device, dtype=torch.float32)
    bias = torch.rand((w.C,), generator=_gen(device, base, 2), device=device, dtype=torch.float32)
    cache = torch.randn((w.B, w.S, w.C), generator=_gen(device, base, 3), device=device,
                        dtype=torch.float32).to(w.torch_dtype)
    return {"x": x, "w": taps * (2 * bound) - bound, "bias": bias * (2 * bound) - bound, "cache": cache}


# ---------------------------------------------------------------------------
# Block-causal softmax attention (the hybrid's periodic softmax blocks).
#
# q [B, H, Tq, S, D], k and v [B, H, Tk, S, D], frame-major like the GDN
# tensors; the queries are the last Tq frames.  Heads and head dim follow the
# 720p-shaped GDN workload (H20, D112, S880); a whole-sequence softmax block
# over all 961 frames is the all-softmax case the pages report running out of
# memory, so the measured clip is 81 frames (the short-clip length) with the
# chunk-causal generator's blocks of 4 frames.  Draw recipe: fp32 ``randn``
# rounded to bf16, one generator per tensor, seeded
# seed * 1_000_003 + 8_000_000 + tensor index (q 0, k 1, v 2).

@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    H: int
    Tq: int
    Tk: int
    S: int
    D: int
    chunk: int

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.Tq * self.S

    def with_(self, **kw) -> "AttnWorkload":
        return dataclasses.replace(self, **kw)


ATTN_CLIP_720P = AttnWorkload("attn-720p-clip B1 H20 T81 S880 D112 chunk4", 1, 20, 81, 81, 880, 112, 4)
ATTN_STREAM_720P = AttnWorkload("attn-720p-stream B1 H20 Tq4 Tk81 S880 D112 chunk4", 1, 20, 4, 81, 880, 112, 4)


def generate_attn(w: AttnWorkload, device="cpu", seed: int = 0) -> Dict[str, torch.Tensor]:
    """q [B, H, Tq, S, D], k and v [B, H, Tk, S, D], bf16."""
    base = seed * 1_000_003 + 8_000_000
    shapes = {"q": (w.B, w.H, w.Tq, w.S, w.D), "k": (w.B, w.H, w.Tk, w.S, w.D), "v": (w.B, w.H, w.Tk, w.S, w.D)}
    return {name: torch.randn(shape, generator=_gen(device, base, i), device=device,
                              dtype=torch.float32).to(torch.bfloat16)
            for i, (name, shape) in enumerate(shapes.items())}

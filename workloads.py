"""Seeded synthetic attention inputs shared by the tests, the smoke check and
the benchmark.

This module holds no attention arithmetic: it only names the workload shapes
and draws their inputs.  Both the GPU path and the CPU oracle consume what it
produces, and neither is imported here.

Recipe (the pages draw Q, K, V with an unseeded standard-normal generator;
here the draw is seeded so both sides see identical bytes):
  g = torch.Generator("cpu").manual_seed(seed)
  q, k, v = torch.randn(B, H, S, D, generator=g, dtype=float32), in that order
  q *= q_mult (a power of two, so the later cast rounds exactly as q would)
  then each is cast to fp16 or bf16 (round to nearest even) and made contiguous.
The softmax scale is fp32(1/sqrt(D)), the value the pages pass explicitly.
"""
from dataclasses import dataclass
import hashlib
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    q_mult: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return softmax_scale(self.D)

    @property
    def torch_dtype(self):
        return torch_dtype(self.dtype)

    def flops(self) -> float:
        """Algorithmic flops, FlashAttention-2 convention: 4*B*H*S^2*D, halved when causal."""
        f = 4.0 * self.B * self.H * self.S * self.S * self.D
        return f / 2 if self.causal else f

    def bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O written once, fp32 lse written."""
        return 4 * self.B * self.H * self.S * self.D * 2 + 4 * self.B * self.H * self.S


# The five workloads: a tiny case, then the attention shapes of the pages' workloads.
WORKLOADS = {
    "tiny_noncausal_1x2x256x64_f16":
        Workload("tiny_noncausal_1x2x256x64_f16", 1, 2, 256, 64, "f16", False, 1.0, 1),
    "gpt_causal_2x12x2048x64_f16":
        Workload("gpt_causal_2x12x2048x64_f16", 2, 12, 2048, 64, "f16", True, 1.0, 2),
    "llama_noncausal_1x32x2048x128_f16":
        Workload("llama_noncausal_1x32x2048x128_f16", 1, 32, 2048, 128, "f16", False, 1.0, 3),
    "long_causal_1x32x8192x128_bf16_q4":
        Workload("long_causal_1x32x8192x128_bf16_q4", 1, 32, 8192, 128, "bf16", True, 4.0, 4),
    "13b_causal_1x40x16384x128_bf16":
        Workload("13b_causal_1x40x16384x128_bf16", 1, 40, 16384, 128, "bf16", True, 1.0, 5),
    # Not one of the five: head dimension 256, which the 2048ai.net page names
    # among the common head dimensions its block size suits (section 3.2);
    # same flops as the long causal case.
    "d256_causal_1x16x8192x256_bf16":
        Workload("d256_causal_1x16x8192x256_bf16", 1, 16, 8192, 256, "bf16", True, 1.0, 6),
}
WORKLOAD_ORDER = list(WORKLOADS)
HEADLINE = "long_causal_1x32x8192x128_bf16_q4"


def torch_dtype(name: str):
    return {"f16": torch.float16, "bf16": torch.bfloat16}[name]


def softmax_scale(D: int) -> float:
    """fp32(1/sqrt(D)) returned as a Python float holding that fp32 value."""
    return float(np.float32(1.0 / math.sqrt(D)))


def make_inputs(B, H, S, D, dtype="f16", seed=0, q_mult=1.0, Sk=None, dist="normal"):
    """Seeded q, k, v CPU tensors of `dtype`, contiguous [B,H,S,D] (k, v: [B,H,Sk,D]).

    dist="normal" is the recipe above; dist="uniform" draws U(-1,1) instead
    (used by tests that need bounded values)."""
    Sk = S if Sk is None else Sk
    g = torch.Generator("cpu").manual_seed(int(seed))
    draw = (lambda *s: torch.randn(*s, generator=g, dtype=torch.float32)) if dist == "normal" \
        else (lambda *s: torch.rand(*s, generator=g, dtype=torch.float32) * 2 - 1)
    q = draw(B, H, S, D)
    k = draw(B, H, Sk, D)
    v = draw(B, H, Sk, D)
    if q_mult != 1.0:
        q = q * q_mult
    td = torch_dtype(dtype)
    return q.to(td).contiguous(), k.to(td).contiguous(), v.to(td).contiguous()


def workload_inputs(w: Workload, seed=None):
    return make_inputs(w.B, w.H, w.S, w.D, w.dtype, w.seed if seed is None else seed, w.q_mult)


def bits(t: torch.Tensor) -> np.ndarray:
    """The 16-bit patterns of a CPU fp16/bf16 tensor as a uint16 numpy array."""
    t = t.detach().contiguous()
    if t.device.type != "cpu":
        t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16)


def sha256(t: torch.Tensor) -> str:
    return hashlib.sha256(bits(t).tobytes()).hexdigest()

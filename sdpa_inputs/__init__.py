"""Seeded synthetic inputs for scaled dot-product attention.

This module is shared by the HIP path's tests and benchmark and by the oracle's
tests. It holds no attention arithmetic: it draws N(0,1) tensors, rounds them
to the storage dtype, and quantises fp8 inputs with a per-tensor amax scale.

Workloads follow the pages' shapes:
  * the first workloads below are the ones the fused kernel is measured and
    checked on (single fp32 head; ViT-B/16 token count 196 with 12 heads of
    64 -- "Self-attention, CUDA kernels and FlashAttention", section 1;
    causal bf16 MHA; causal GQA/MQA with shared KV heads -- codelab
    "Accelerate attention on GPU with cuDNN and TransformerEngine", section 9;
    and a long causal fp8-e4m3 workload -- same codelab, section 10); then a
    decode step (one query per sequence against a long KV cache, GQA heads of
    section 9) for the split-KV path, and the causal GQA shape's backward pass;
  * every draw is i.i.d. standard normal, as every input cell of the codelab
    is (sections 3, 8, 9, 10), and bf16 values are fp32 draws cast to bf16
    (section 6).

Seeds follow the codelab's PRNG key numbers (key 0 for the default arrays,
the sequence length for the sweep, 42 for the MHA/GQA/MQA cell, 9000 for the
FP8 cell, sequence length + 1000 for the causal sweep). The streams are numpy
PCG64 streams, not JAX threefry: values differ from the codelab's.

Layout is [B, H, S, d] row-major for every tensor (the layout the codelab's
from-scratch attention transposes its (B, T, N, H) arrays into, section 4).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

E4M3_MAX = 448.0  # largest finite OCP e4m3fn magnitude
E5M2_MAX = 57344.0  # largest finite OCP e5m2 magnitude

DTYPES = ("f32", "bf16", "fp8")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    d: int
    dtype: str  # "f32" | "bf16" | "fp8" (e4m3fn inputs, bf16 output)
    causal: bool
    seed: int
    want_lse: bool = False
    path: str = "fused"  # "fused": attn_fwd / attn_fwd_fp8; "splitkv": attn_fwd_splitkv; "bwd": attn_bwd

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Causal-adjusted algorithmic FLOP: 4*B*Hq*Sq*Sk*d, halved when causal (two
        Sq x Sk x d products). The backward pass has five such products (S, dP, dV,
        dK, dQ; recomputation not counted): 2.5 times the forward."""
        f = 4.0 * self.B * self.Hq * self.Sq * self.Sk * self.d
        if self.path == "bwd":
            f *= 2.5
        return f * 0.5 if self.causal else f

    def hbm_bytes(self) -> float:
        """Algorithmic HBM bytes: Q, K, V read once; O (and LSE) written once."""
        ein = {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]
        eout = {"f32": 4, "bf16": 2, "fp8": 2}[self.dtype]
        q = self.B * self.Hq * self.Sq * self.d * ein
        kv = 2 * self.B * self.Hkv * self.Sk * self.d * ein
        o = self.B * self.Hq * self.Sq * self.d * eout
        lse = self.B * self.Hq * self.Sq * 4 if self.want_lse else 0
        if self.path == "bwd":
            # reads Q, K, V, O, dO and lse once; writes dQ, dK, dV once
            return float(2 * q + 2 * kv + 2 * o + self.B * self.Hq * self.Sq * 4)
        return float(q + kv + o + lse)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("single_head_f32_s128_d64", 1, 1, 1, 128, 128, 64, "f32", False, 0),
        Workload("vit_b16_bf16_b32_h12_s196_d64", 32, 12, 12, 196, 196, 64, "bf16", False, 196),
        Workload("causal_mha_bf16_b8_h16_s2048_d128", 8, 16, 16, 2048, 2048, 128, "bf16", True, 3048,
                 want_lse=True),
        Workload("causal_gqa_bf16_b4_hq32_hkv8_s4096_d128", 4, 32, 8, 4096, 4096, 128, "bf16", True, 42),
        Workload("causal_mqa_bf16_b4_hq32_hkv1_s4096_d128", 4, 32, 1, 4096, 4096, 128, "bf16", True, 42),
        Workload("causal_fp8_b1_h32_s16384_d128", 1, 32, 32, 16384, 16384, 128, "fp8", True, 9000),
        # One new token per sequence against a 32K-token KV cache, the GQA cell's head layout.
        Workload("decode_gqa_bf16_b4_hq32_hkv8_sk32768_d128", 4, 32, 8, 1, 32768, 128, "bf16", False, 42,
                 path="splitkv"),
        # The headline shape's backward pass (dQ, dK, dV from the forward's O and lse and a seeded dO).
        Workload("bwd_causal_gqa_bf16_b4_hq32_hkv8_s4096_d128", 4, 32, 8, 4096, 4096, 128, "bf16", True, 42,
                 path="bwd"),
    ]
}

# The workload the headline throughput is quoted on.
HEADLINE = "causal_gqa_bf16_b4_hq32_hkv8_s4096_d128"


def _normal(seq: np.random.SeedSequence, shape) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seq)).standard_normal(shape, dtype=np.float32)


def draw_qkv(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int, seed: int):
    """Draw fp32 N(0,1) Q [B,Hq,Sq,d], K and V [B,Hkv,Sk,d] from one seed.

    Q depends only on (seed, shape of Q), so workloads that differ only in the
    number of KV heads share the same queries; K and V streams also fold in
    Hkv. Returns three float32 torch CPU tensors.
    """
    q = _normal(np.random.SeedSequence([seed, 0]), (B, Hq, Sq, d))
    k = _normal(np.random.SeedSequence([seed, 1, Hkv]), (B, Hkv, Sk, d))
    v = _normal(np.random.SeedSequence([seed, 2, Hkv]), (B, Hkv, Sk, d))
    return torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)


def quantise_e4m3(x: torch.Tensor):
    """Per-tensor amax quantisation of fp32 ``x`` to OCP fp8-e4m3fn.

    scale = 448 / amax(|x|) in fp32; codes = RNE(x * scale) saturated to
    +-448; descale = 1 / scale in fp32. Returns (codes as uint8 tensor,
    descale as a Python float holding the exact fp32 value).
    """
    x = x.to(torch.float32)
    amax = float(x.abs().max())
    if not math.isfinite(amax) or amax == 0.0:
        amax = 1.0
    s = torch.tensor(E4M3_MAX, dtype=torch.float32) / torch.tensor(amax, dtype=torch.float32)
    y = torch.clamp(x * s, -E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    descale = float((torch.tensor(1.0, dtype=torch.float32) / s).item())
    return codes.contiguous(), descale


def quantise_e5m2(x: torch.Tensor):
    """Per-tensor amax quantisation of fp32 ``x`` to OCP fp8-e5m2, the gradient
    format of the codelab's fp8 recipe (section 10).

    scale = 57344 / amax(|x|) in fp32; codes = RNE(x * scale) saturated to
    +-57344 (never infinity); descale = 1 / scale in fp32. Returns (codes as
    uint8 tensor, descale as a Python float holding the exact fp32 value).
    """
    x = x.to(torch.float32)
    amax = float(x.abs().max())
    if not math.isfinite(amax) or amax == 0.0:
        amax = 1.0
    s = torch.tensor(E5M2_MAX, dtype=torch.float32) / torch.tensor(amax, dtype=torch.float32)
    y = torch.clamp(x * s, -E5M2_MAX, E5M2_MAX)
    codes = y.to(torch.float8_e5m2).view(torch.uint8)
    descale = float((torch.tensor(1.0, dtype=torch.float32) / s).item())
    return codes.contiguous(), descale


def draw_grad_fp8(w: Workload, seed: Optional[int] = None):
    """The upstream gradient of draw_grad's stream as fp8-e5m2 codes with a
    per-tensor descale: (codes uint8 [B, Hq, Sq, d], descale)."""
    seed = w.seed if seed is None else seed
    g = _normal(np.random.SeedSequence([seed, 3]), (w.B, w.Hq, w.Sq, w.d))
    return quantise_e5m2(torch.from_numpy(g))


def draw_grad(w: Workload, seed: Optional[int] = None) -> torch.Tensor:
    """A seeded upstream gradient dL/dO for the backward pass: N(0,1) of O's
    shape [B, Hq, Sq, d], rounded to bf16 (its own stream of the workload's seed)."""
    seed = w.seed if seed is None else seed
    g = _normal(np.random.SeedSequence([seed, 3]), (w.B, w.Hq, w.Sq, w.d))
    return torch.from_numpy(g).to(torch.bfloat16)


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Inputs for workload ``w`` as torch CPU tensors in the storage dtype.

    Returns a dict with q, k, v (float32, bfloat16, or uint8 e4m3fn codes) and,
    for fp8, descale_q/k/v (fp32 values as Python floats; 1.0 otherwise).
    """
    seed = w.seed if seed is None else seed
    q, k, v = draw_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d, seed)
    out = {"descale_q": 1.0, "descale_k": 1.0, "descale_v": 1.0}
    if w.dtype == "f32":
        out.update(q=q, k=k, v=v)
    elif w.dtype == "bf16":
        out.update(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16), v=v.to(torch.bfloat16))
    elif w.dtype == "fp8":
        for name, t in (("q", q), ("k", k), ("v", v)):
            codes, ds = quantise_e4m3(t)
            out[name] = codes
            out["descale_" + name] = ds
    else:
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return out


def custom(B, Hq, Hkv, Sq, Sk, d, dtype, causal, seed, want_lse=False, name=None) -> Workload:
    """A workload of any shape (tests use these for tails and edge cases)."""
    return Workload(name or f"custom_{dtype}_b{B}_hq{Hq}_hkv{Hkv}_sq{Sq}_sk{Sk}_d{d}_{'c' if causal else 'n'}",
                    B, Hq, Hkv, Sq, Sk, d, dtype, causal, seed, want_lse)

"""Plain fp64 CPU definition of scaled dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module:
only tests, the smoke check and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP kernels.

What it computes (codelab "Accelerate attention on GPU with cuDNN and
TransformerEngine", intro "How attention works" and section 4; article
"Self-attention, CUDA kernels and FlashAttention", section 1): for every batch
b, query head h and query row i,

  1. score    s_j = scale * <Q[b,h,i,:], K[b,hk,j,:]>   for each allowed key j
  2. softmax  w_j = exp(s_j - max s) / sum_l exp(s_l - max s)   (rows sum to 1)
  3. attend   O[b,h,i,:] = sum_j w_j V[b,hk,j,:]         (O has Q's shape)
  4. stats    lse[b,h,i] = max s + ln sum_j exp(s_j - max s)

where
  * allowed keys are all j in [0, Sk), or j <= i + (Sk - Sq) under the causal
    mask. With Sq == Sk this is the codelab's lower-triangular mask (section 7:
    the first position sees only itself, the last sees every position). With
    Sq < Sk the queries are the last Sq positions of the key sequence, as when
    new tokens attend to a KV cache (codelab section 9): the last query still
    sees every key (bottom-right alignment; the pages fix no rule for Sq != Sk,
    this is the reading that keeps their first/last-position statement). Sq >
    Sk under the mask would leave rows with no key and is rejected;
  * hk = h // (Hq // Hkv): consecutive query heads share one KV head
    (codelab section 9: fewer KV heads are broadcast over the query heads,
    e.g. 2 KV heads each serving 4 of 8 query heads);
  * lse is the per-row normalisation statistic the article's section 3 says a
    fused kernel keeps for the backward pass, in natural-log units.

Subtracting the row maximum before exp is an identity of softmax and keeps
large-offset inputs finite. The FlashAttention restructuring (tiles plus an
online softmax, article section 3) reaches this same result up to rounding,
so the oracle is the plain definition, row by row; rows are independent, so
computing them in blocks changes no value.
"""

from __future__ import annotations

from typing import Iterable, Tuple

import numpy as np


def _check(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool) -> Tuple[int, int, int, int, int, int]:
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, d]")
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if k.shape != v.shape or Bk != B or dk != d:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    if causal and Sq > Sk:
        raise ValueError("under the causal mask the first Sq - Sk query rows would see no key (Sq > Sk)")
    return B, Hq, Hkv, Sq, Sk, d


def attention_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   row_index: np.ndarray, causal: bool, key_offset: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Attention for selected query rows of ONE (batch, head).

    q_rows [R, d] are the query vectors, row_index [R] their positions in the
    query sequence (used only by the causal mask, which lets row i see keys
    j <= i + key_offset), k and v [Sk, d] that head's keys and values.
    Returns (O [R, d], lse [R]) in fp64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    # step 1: scores
    s = (q_rows @ k.T) * float(scale)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j <= np.asarray(row_index)[:, None] + int(key_offset), s, -np.inf)
    # step 2: softmax over the allowed keys of each row
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    w = e / den
    # step 3: weighted sum of values
    o = w @ v
    # step 4: log of the normaliser, natural-log units
    lse = m[:, 0] + np.log(den[:, 0])
    return o, lse


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
              row_block: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Full attention: q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] -> (O [B,Hq,Sq,d], lse [B,Hq,Sq]), fp64."""
    B, Hq, Hkv, Sq, Sk, d = _check(q, k, v, causal)
    G = Hq // Hkv
    o = np.empty((B, Hq, Sq, d), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i0 in range(0, Sq, row_block):
                i1 = min(Sq, i0 + row_block)
                o[b, h, i0:i1], lse[b, h, i0:i1] = attention_rows(
                    q[b, h, i0:i1], k[b, hk], v[b, hk], scale, np.arange(i0, i1), causal, Sk - Sq)
    return o, lse


def attention_sampled(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool,
                      samples: Iterable[Tuple[int, int, np.ndarray]]):
    """Attention at sampled positions only.

    ``samples`` yields (b, h, rows) with rows an int array of query positions.
    Returns a list of (b, h, rows, O [R, d], lse [R]) in fp64. Used where the
    full problem is too large for the CPU: each sampled row is computed
    exactly as in :func:`attention`.
    """
    B, Hq, Hkv, Sq, Sk, d = _check(q, k, v, causal)
    G = Hq // Hkv
    out = []
    for b, h, rows in samples:
        rows = np.asarray(rows, dtype=np.int64)
        o, lse = attention_rows(q[b, h, rows], k[b, h // G], v[b, h // G], scale, rows, causal, Sk - Sq)
        out.append((b, h, rows, o, lse))
    return out

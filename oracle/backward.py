"""Plain fp64 CPU definition of the gradients of scaled dot-product attention.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the product path never
imports it, and it shares no code with the HIP kernels.

What it computes. The forward pass is oracle.attention: for each (b, h) and
query row i, over the allowed keys j,

    s_ij = scale * <Q_i, K_j>,   P_ij = exp(s_ij - lse_i),   O_i = sum_j P_ij V_j.

Given the gradient dO = dL/dO of some scalar loss L, the gradients with respect
to Q, K and V follow from the chain rule through the codelab's three steps
("Accelerate attention on GPU with cuDNN and TransformerEngine", section 4:
score, softmax, weighted sum), taken in reverse order:

    attend:   dV_j  = sum_i P_ij dO_i             dP_ij = <dO_i, V_j>
    softmax:  dS_ij = P_ij (dP_ij - sum_l P_il dP_il)   (the softmax Jacobian)
    score:    dQ_i  = scale sum_j dS_ij K_j       dK_j  = scale sum_i dS_ij Q_i

Masked (key, query) pairs have P_ij = 0 and add nothing. A KV head read by
several query heads (GQA/MQA, codelab section 9) receives the sum of their
gradients. The article "Self-attention, CUDA kernels and FlashAttention"
(section 3) describes the fused backward pass as recomputing P from the stored
per-row statistic instead of keeping the N x N matrix; that changes where P
comes from, not these values, so the oracle is the plain definition: P from
the forward oracle's definition, row blocks computed independently.
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import _check


def _weights(q_rows: np.ndarray, k: np.ndarray, scale: float, rows: np.ndarray, causal: bool,
             key_offset: int) -> np.ndarray:
    """P [R, Sk] of one (batch, head): softmax over the allowed keys of each row."""
    s = (q_rows @ k.T) * float(scale)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j <= rows[:, None] + int(key_offset), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=1, keepdims=True)


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                       causal: bool = False, row_block: int = 512) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dQ [B,Hq,Sq,d], dK [B,Hkv,Sk,d], dV [B,Hkv,Sk,d]) in fp64 for the loss gradient ``do`` [B,Hq,Sq,d].

    The causal mask and the head mapping are those of oracle.attention (query i
    sees keys j <= i + Sk - Sq; query head h reads KV head h // (Hq // Hkv)).
    """
    B, Hq, Hkv, Sq, Sk, d = _check(q, k, v, causal)
    if do.shape != q.shape:
        raise ValueError(f"dO {do.shape} must have Q's shape {q.shape}")
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    G = Hq // Hkv
    dq = np.zeros((B, Hq, Sq, d))
    dk = np.zeros((B, Hkv, Sk, d))
    dv = np.zeros((B, Hkv, Sk, d))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            kk, vv = k[b, hk], v[b, hk]
            for i0 in range(0, Sq, row_block):
                i1 = min(Sq, i0 + row_block)
                rows = np.arange(i0, i1)
                p = _weights(q[b, h, i0:i1], kk, scale, rows, causal, Sk - Sq)
                g = do[b, h, i0:i1]
                # attend, reversed
                dv[b, hk] += p.T @ g
                dp = g @ vv.T
                # softmax, reversed: the Jacobian applied row by row
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                # score, reversed
                dq[b, h, i0:i1] = float(scale) * (ds @ kk)
                dk[b, hk] += float(scale) * (ds.T @ q[b, h, i0:i1])
    return dq, dk, dv

"""Helpers of the GPU parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same seeded inputs, then compare element by element."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from oracle import e4m3
import sdpa_inputs

# Tolerances: max |GPU - oracle| over every compared element. O: fixed per dtype.
# lse: the bf16 and fp8 kernels sum the bf16-rounded probabilities that the
# P.V product consumes (relative error <= 2^-8 each), so their log-sum-exp can
# be off by up to ln(1 + 2^-8) = 3.9e-3; the fp32 kernel keeps fp32 probabilities.
TOL_O = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
TOL_LSE = {"f32": 1e-4, "bf16": 4e-3, "fp8": 1e-2}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp: dict) -> dict:
    out = dict(inp)
    for n in ("q", "k", "v"):
        out[n] = inp[n].cuda()
    return out


def run_gpu(w: sdpa_inputs.Workload, dev: dict, want_lse: bool = True, out=None, lse_out=None):
    import scaled_dot_product_18_amd as sdpa
    if w.dtype == "fp8":
        o, lse = sdpa.fwd_fp8(dev["q"], dev["k"], dev["v"], dev["descale_q"], dev["descale_k"], dev["descale_v"],
                              causal=w.causal, scale=w.scale, want_lse=want_lse, out=out, lse_out=lse_out)
    else:
        o, lse = sdpa.fwd(dev["q"], dev["k"], dev["v"], causal=w.causal, scale=w.scale, want_lse=want_lse,
                          out=out, lse_out=lse_out)
    return o, lse


def oracle_arrays(w: sdpa_inputs.Workload, inp: dict):
    """fp64 numpy copies of the exact values the GPU receives."""
    if w.dtype == "fp8":
        return tuple(oracle.dequantise(e4m3.decode(inp[n].numpy()), inp["descale_" + n]) for n in ("q", "k", "v"))
    return tuple(inp[n].to(torch.float64).numpy() for n in ("q", "k", "v"))


def check_full(w, inp, o_gpu, lse_gpu):
    """Element-by-element comparison against the full oracle."""
    q, k, v = oracle_arrays(w, inp)
    o_ref, lse_ref = oracle.attention(q, k, v, w.scale, w.causal)
    o = o_gpu.to(torch.float64).cpu().numpy()
    assert np.isfinite(o).all(), f"{w.name}: non-finite output"
    err = np.abs(o - o_ref)
    stats = {"max_err_o": float(err.max()), "mean_err_o": float(err.mean())}
    if lse_gpu is not None:
        lse = lse_gpu.to(torch.float64).cpu().numpy()
        assert np.isfinite(lse).all(), f"{w.name}: non-finite lse"
        stats["max_err_lse"] = float(np.abs(lse - lse_ref).max())
    assert stats["max_err_o"] <= TOL_O[w.dtype], f"{w.name}: {stats}"
    if lse_gpu is not None:
        assert stats["max_err_lse"] <= TOL_LSE[w.dtype], f"{w.name}: {stats}"
    return stats


def sample_rows(S: int, rng: np.random.Generator, n_random: int = 24, block: int = 128) -> np.ndarray:
    """First rows (where causal softmax is sharpest), tile edges, the last rows and random rows."""
    fixed = [0, 1, 2, 3, 7, S - 1, S - 2, S // 2]
    for t in range(block, S, block * max(1, (S // block) // 4)):
        fixed += [t - 1, t, t + 1]
    rows = set(r for r in fixed if 0 <= r < S)
    rows.update(rng.choice(S, size=min(S, n_random), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def check_sampled(w, inp, o_gpu, lse_gpu, heads=None, n_random: int = 24, seed: int = 7):
    """Compare sampled rows of every (b, h) (or of ``heads``) with the oracle row by row."""
    rng = np.random.default_rng(seed)
    o = o_gpu.to(torch.float32).cpu()
    lse = lse_gpu.cpu() if lse_gpu is not None else None
    G = w.Hq // w.Hkv
    if w.dtype == "fp8":
        dq, dk, dv = inp["descale_q"], inp["descale_k"], inp["descale_v"]
        conv = {"q": lambda t: e4m3.decode(t.numpy()) * dq, "k": lambda t: e4m3.decode(t.numpy()) * dk,
                "v": lambda t: e4m3.decode(t.numpy()) * dv}
    else:
        conv = {n: (lambda t: t.to(torch.float64).numpy()) for n in ("q", "k", "v")}
    worst_o, worst_l, n_rows = 0.0, 0.0, 0
    kv_cache = {}
    for b in range(w.B):
        for h in (range(w.Hq) if heads is None else heads):
            hk = h // G
            if (b, hk) not in kv_cache:
                kv_cache.clear()
                kv_cache[(b, hk)] = (conv["k"](inp["k"][b, hk]), conv["v"](inp["v"][b, hk]))
            kk, vv = kv_cache[(b, hk)]
            rows = sample_rows(w.Sq, rng, n_random)
            qq = conv["q"](inp["q"][b, h][torch.from_numpy(rows)])
            o_ref, l_ref = oracle.attention_rows(qq, kk, vv, w.scale, rows, w.causal)
            got = o[b, h][torch.from_numpy(rows)].to(torch.float64).numpy()
            assert np.isfinite(got).all()
            worst_o = max(worst_o, float(np.abs(got - o_ref).max()))
            if lse is not None:
                gl = lse[b, h][torch.from_numpy(rows)].to(torch.float64).numpy()
                worst_l = max(worst_l, float(np.abs(gl - l_ref).max()))
            n_rows += len(rows)
    stats = {"max_err_o": worst_o, "max_err_lse": worst_l if lse is not None else None, "rows": n_rows}
    assert worst_o <= TOL_O[w.dtype], f"{w.name}: {stats}"
    if lse is not None:
        assert worst_l <= TOL_LSE[w.dtype], f"{w.name}: {stats}"
    return stats

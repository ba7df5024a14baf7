"""Helpers of the GPU parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same seeded inputs, then compare element by element."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from oracle import e4m3
import sdpa_inputs

# Tolerances: max |GPU - oracle| over every compared element. O: fixed per dtype
# (1e-4 fp32, 2e-2 bf16, 6e-2 fp8 on dequantised inputs), plus p8_bound below
# for the fp8 rows whose P.V takes P rounded to e4m3.
# lse: every kernel adds the unrounded fp32 probabilities into its row sum (the
# bf16 rounding of P only feeds the P.V product), so lse = ln 2 (m + log2 l)
# carries only fp32 error: scores of exactly representable inputs accumulated in
# fp32 (|s| <= ~10 here, d <= 128 terms: ~1e-6), exp2 to ~2 ulp, and a row sum of
# up to 16384 terms, added into a few fp32 partials (relative error <= ~2^-24
# per add, < 2e-5 for the longest rows). 1e-4 holds every path with margin;
# tests with scores of order 1e3 add 1e-5 |lse| for the fp32 rounding of the scores.
TOL_O = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
TOL_LSE = {"f32": 1e-4, "bf16": 1e-4, "fp8": 1e-3}


# The fp8 d = 128 kernel runs P.V on fp8 matrix cores (P rounded to e4m3) for
# the 256-row q-tiles whose first query sees at least 256 keys, and on bf16
# matrix cores for the others (its launcher's rule, mirrored here).
P8_TILE = 256
LOG2E = 1.4426950408889634


def key_half_d128(w) -> bool:
    """d = 128 shapes the key-half kernel takes: at most 256 q-tiles of 128 rows
    over all heads and batches, 512 under the causal mask."""
    return w.d == 128 and (w.Sq + 127) // 128 * w.B * w.Hq <= (512 if w.causal else 256)


def p8_first_row(w):
    """First query row whose P.V runs with P in e4m3, or None if no row does
    (only the 256-row d = 128 fp8 kernel rounds P to e4m3; the key-half kernel,
    whose P is bf16, takes the small shapes)."""
    if w.dtype != "fp8" or w.d != 128 or key_half_d128(w):
        return None
    n_qt = (w.Sq + P8_TILE - 1) // P8_TILE
    if not w.causal:
        first = 0 if w.Sk >= P8_TILE else n_qt
    else:
        need = P8_TILE - 1 - (w.Sk - w.Sq)
        first = 0 if need <= 0 else (need + P8_TILE - 1) // P8_TILE
    return first * P8_TILE if first < n_qt else None


def p8_bound(q_rows, k, v, scale, rows, causal, key_offset, lse_rows, chunk=256):
    """Per-element bound [R, d] of the extra error of P.V with P rounded to e4m3,
    from the exact softmax weights w_ij = exp(s_ij - lse_i) (lse from the oracle).
    The kernel stores 2 P_ij = 2^(log2e (s_ij - m) + 1) with a reference m no
    larger than the row maximum: while that is a normal e4m3 value its rounding
    is at most 2^-4 of it; it can be subnormal only if log2e (s_ij - max_i) < -7,
    and then the bound takes all of it. With l the fp32 sum of the unrounded P,
    |dO_ic| <= 2^-4 sum_{j not in S_i} w_ij |V_jc| + sum_{j in S_i} w_ij |V_jc|,
    S_i = {j : log2e (s_ij - max_i) < -6.5} (half a binade of margin for the
    kernel's fp32 scores)."""
    absv = np.abs(v)
    out = np.empty((len(rows), v.shape[1]))
    cols = np.arange(k.shape[0])
    for c0 in range(0, len(rows), chunk):
        sl = slice(c0, c0 + chunk)
        s = scale * (q_rows[sl] @ k.T)
        if causal:
            s = np.where(cols[None, :] <= rows[sl, None] + key_offset, s, -np.inf)
        wgt = np.exp(s - lse_rows[sl, None])
        small = LOG2E * (s - s.max(axis=1, keepdims=True)) < -6.5
        out[sl] = 2.0 ** -4 * (np.where(small, 0.0, wgt) @ absv) + np.where(small, wgt, 0.0) @ absv
    return out


def kernel_block_m(w) -> int:
    """Query rows per head of one workgroup of the kernel the launcher picks for
    ``w``: the d = 128 bf16 and fp8 kernels take 256-row tiles, the others 128;
    the causal d = 128 bf16 kernel packs 4 (2) query heads of one KV head into
    a workgroup when the group size divides by 4 (2), 64 (128) rows each. Small
    d = 128 bf16 and fp8 shapes run the key-half kernel on 128-row tiles instead."""
    if w.dtype in ("bf16", "fp8") and key_half_d128(w):
        return 128
    if w.d == 128 and w.dtype == "bf16":
        G = w.Hq // w.Hkv
        return 256 // (1 if not w.causal else 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1)
    return 256 if (w.d == 128 and w.dtype == "fp8") else 128


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
        return tuple(e4m3.dequantise(inp[n].numpy(), inp["descale_" + n]) for n in ("q", "k", "v"))
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
    tol = np.full(err.shape, TOL_O[w.dtype])
    first = p8_first_row(w)
    if first is not None:
        G = w.Hq // w.Hkv
        rows = np.arange(first, w.Sq)
        for b in range(w.B):
            for h in range(w.Hq):
                tol[b, h, first:] += p8_bound(q[b, h, first:], k[b, h // G], v[b, h // G], w.scale, rows, w.causal,
                                              w.Sk - w.Sq if w.causal else 0, lse_ref[b, h, first:])
        stats["p8_rows_from"] = first
        stats["max_err_over_tol"] = float((err / tol).max())
    assert (err <= tol).all(), f"{w.name}: {stats}"
    if lse_gpu is not None:
        assert stats["max_err_lse"] <= TOL_LSE[w.dtype], f"{w.name}: {stats}"
    return stats


def sample_rows(S: int, rng: np.random.Generator, n_random: int = 24, block: int = 128,
                first: int = 8) -> np.ndarray:
    """The first ``first`` rows (where causal softmax is sharpest), rows at tile
    edges of ``block`` rows, the last rows and ``n_random`` random rows."""
    fixed = list(range(min(S, first))) + [S - 1, S - 2, S // 2]
    for t in range(block, S, block * max(1, (S // block) // 4)):
        fixed += [t - 1, t, t + 1]
    rows = set(r for r in fixed if 0 <= r < S)
    rows.update(rng.choice(S, size=min(S, n_random), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def check_sampled(w, inp, o_gpu, lse_gpu, heads=None, n_random: int = 24, seed: int = 7, first: int = 8):
    """Compare sampled rows of every (b, h) (or of ``heads``) with the oracle row by row:
    see sample_rows; tile edges sit at the launched kernel's q-tile size."""
    rng = np.random.default_rng(seed)
    o = o_gpu.to(torch.float32).cpu()
    lse = lse_gpu.cpu() if lse_gpu is not None else None
    G = w.Hq // w.Hkv
    if w.dtype == "fp8":
        conv = {n: (lambda t, n=n: e4m3.dequantise(t.numpy(), inp["descale_" + n])) for n in ("q", "k", "v")}
    else:
        conv = {n: (lambda t: t.to(torch.float64).numpy()) for n in ("q", "k", "v")}
    key_offset = w.Sk - w.Sq if w.causal else 0
    block = kernel_block_m(w)
    worst_o, worst_l, n_rows, sum_err, n_el, worst_ratio = 0.0, 0.0, 0, 0.0, 0, 0.0
    first_p8 = p8_first_row(w)
    kv_cache = {}
    for b in range(w.B):
        for h in (range(w.Hq) if heads is None else heads):
            hk = h // G
            if (b, hk) not in kv_cache:
                kv_cache.clear()
                kv_cache[(b, hk)] = (conv["k"](inp["k"][b, hk]), conv["v"](inp["v"][b, hk]))
            kk, vv = kv_cache[(b, hk)]
            rows = sample_rows(w.Sq, rng, n_random, block=block, first=first)
            qq = conv["q"](inp["q"][b, h][torch.from_numpy(rows)])
            o_ref, l_ref = oracle.attention_rows(qq, kk, vv, w.scale, rows, w.causal, key_offset)
            got = o[b, h][torch.from_numpy(rows)].to(torch.float64).numpy()
            assert np.isfinite(got).all()
            err = np.abs(got - o_ref)
            tol = np.full(err.shape, TOL_O[w.dtype])
            if first_p8 is not None and (rows >= first_p8).any():
                sel = rows >= first_p8
                tol[sel] += p8_bound(qq[sel], kk, vv, w.scale, rows[sel], w.causal, key_offset, l_ref[sel])
            assert (err <= tol).all(), f"{w.name}: b {b} h {h}: max err {err.max()}, max err/tol {(err / tol).max()}"
            worst_ratio = max(worst_ratio, float((err / tol).max()))
            worst_o = max(worst_o, float(err.max()))
            sum_err += float(err.sum())
            n_el += err.size
            if lse is not None:
                gl = lse[b, h][torch.from_numpy(rows)].to(torch.float64).numpy()
                worst_l = max(worst_l, float(np.abs(gl - l_ref).max()))
            n_rows += len(rows)
    stats = {"max_err_o": worst_o, "mean_err_o": sum_err / max(1, n_el),
             "max_err_lse": worst_l if lse is not None else None, "rows": n_rows, "max_err_over_tol": worst_ratio,
             "p8_rows_from": first_p8}
    if lse is not None:
        assert worst_l <= TOL_LSE[w.dtype], f"{w.name}: {stats}"
    return stats

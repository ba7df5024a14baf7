"""GPU parity of the backward pass (attn_bwd) against the fp64 gradient oracle.

The HIP forward produces O and lse, the HIP backward takes them with a seeded
upstream gradient dO, and dQ, dK, dV are compared element by element with
oracle.attention_backward on the same bf16 values. Tolerance (no figure on the
pages; derived from the arithmetic): P and dS enter the matrix cores rounded
to bf16 (relative error 2^-9 each) and the gradients are stored in bf16, so the
error is a few 2^-9 of the gradient's own scale; the test allows
max|GPU - oracle| <= 2e-2 * max(1, max|oracle|) per tensor.
"""

import itertools

import numpy as np
import pytest
import torch

from oracle.backward import attention_backward
import sdpa_inputs
from parity_util import log

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _run(w):
    import scaled_dot_product_18_amd as sdpa
    log(f"[bwd] {w.name}")
    inp = sdpa_inputs.make_inputs(w)
    g = sdpa_inputs.draw_grad(w)
    q, k, v, do = (t.cuda() for t in (inp["q"], inp["k"], inp["v"], g))
    o, lse = sdpa.fwd(q, k, v, causal=w.causal, scale=w.scale, want_lse=True)
    dq, dk, dv = sdpa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    ref = attention_backward(*(t.to(torch.float64).numpy() for t in (inp["q"], inp["k"], inp["v"], g)),
                             w.scale, w.causal)
    stats = {}
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        x = got.to(torch.float64).cpu().numpy()
        assert np.isfinite(x).all(), f"{w.name}: non-finite {name}"
        err = float(np.abs(x - r).max())
        scale = max(1.0, float(np.abs(r).max()))
        stats[name] = (round(err, 5), round(scale, 3))
        assert err <= TOL * scale, f"{w.name}: {name} max err {err} (scale {scale}) {stats}"
    return stats, (dq, dk, dv), (q, k, v, o, lse, do)


S_LIST = [1, 17, 64, 65, 128, 129, 200, 257]
HEADS = [(4, 4), (4, 2), (4, 1)]


@pytest.mark.parametrize("S,d,causal,heads", list(itertools.product(S_LIST, (64, 128), (False, True), HEADS)))
def test_bwd_tails(gpu, S, d, causal, heads):
    Hq, Hkv = heads
    stats, *_ = _run(sdpa_inputs.custom(1, Hq, Hkv, S, S, d, "bf16", causal, seed=11000 + S))
    log(f"  {stats}")


# Groups of 8 and 16 query heads per KV head: the dK/dV kernel splits them into
# 2 and 4 subsets whose fp32 partial sums a second kernel adds.
SPLIT_HEADS = [(8, 1), (16, 1), (16, 2)]


@pytest.mark.parametrize("S,d,causal,heads", list(itertools.product([17, 129, 257], (64, 128), (False, True),
                                                                    SPLIT_HEADS)))
def test_bwd_query_head_subsets(gpu, S, d, causal, heads):
    Hq, Hkv = heads
    stats, *_ = _run(sdpa_inputs.custom(2, Hq, Hkv, S, S, d, "bf16", causal, seed=14000 + S + Hq))
    log(f"  {stats}")


@pytest.mark.parametrize("Sq,Sk,d", [(1, 300, 128), (5, 64, 64), (77, 200, 128), (130, 257, 64), (256, 1000, 128)])
def test_bwd_queries_are_the_last_positions(gpu, Sq, Sk, d):
    """Causal with Sq < Sk (bottom-right mask), and the same shapes unmasked."""
    for causal in (True, False):
        _run(sdpa_inputs.custom(2, 4, 2, Sq, Sk, d, "bf16", causal, seed=12000 + Sq + Sk))


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_batches_and_groups(gpu, d):
    stats, *_ = _run(sdpa_inputs.custom(3, 12, 3, 300, 300, d, "bf16", True, seed=13000 + d))
    log(f"  {stats}")


def test_bwd_is_deterministic(gpu):
    """No atomics: two calls give identical bits."""
    import scaled_dot_product_18_amd as sdpa
    _, first, (q, k, v, o, lse, do) = _run(sdpa_inputs.custom(2, 8, 2, 333, 333, 128, "bf16", True, seed=14000))
    second = sdpa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)


def test_bwd_errors_raise_through_python(gpu):
    import scaled_dot_product_18_amd as sdpa
    z = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 2, 8, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):  # mixed dtypes
        sdpa.bwd(z.float(), z, z, z, lse, z)
    with pytest.raises(ValueError):  # fp16 is not a backward dtype
        sdpa.bwd(z.half(), z.half(), z.half(), z.half(), lse, z.half())
    with pytest.raises(ValueError):
        sdpa.bwd(z, z, z, z, lse[:, :, :4].contiguous(), z)
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.bwd(z, z, z, z, lse, z, workspace=torch.empty(8, dtype=torch.uint8, device="cuda"))
    assert e.value.status == -10


def test_bwd_benchmark_workload_sampled_groups(gpu):
    """The benchmark's backward workload (causal GQA B4 Hq32 Hkv8 S4096 d128), launched as the
    benchmark launches it; two whole KV-head groups (their 4 query heads' dQ and the KV head's dK,
    dV: every element) are compared with the oracle run on that group alone."""
    import scaled_dot_product_18_amd as sdpa
    w = sdpa_inputs.WORKLOADS["bwd_causal_gqa_bf16_b4_hq32_hkv8_s4096_d128"]
    assert w.path == "bwd"
    log(f"[bwd-full] {w.name}")
    inp = sdpa_inputs.make_inputs(w)
    g = sdpa_inputs.draw_grad(w)
    q, k, v, do = (t.cuda() for t in (inp["q"], inp["k"], inp["v"], g))
    o, lse = sdpa.fwd(q, k, v, causal=True, scale=w.scale, want_lse=True)
    dq, dk, dv = sdpa.bwd(q, k, v, o, lse, do, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    for b, hk in [(0, 0), (w.B - 1, w.Hkv - 1)]:
        hs = slice(hk * G, (hk + 1) * G)
        ref = attention_backward(inp["q"][b:b + 1, hs].double().numpy(), inp["k"][b:b + 1, hk:hk + 1].double().numpy(),
                                 inp["v"][b:b + 1, hk:hk + 1].double().numpy(), g[b:b + 1, hs].double().numpy(),
                                 w.scale, True)
        for name, got, r in zip(("dq", "dk", "dv"), (dq[b:b + 1, hs], dk[b:b + 1, hk:hk + 1], dv[b:b + 1, hk:hk + 1]),
                                ref):
            x = got.double().cpu().numpy()
            err = float(np.abs(x - r).max())
            scale = max(1.0, float(np.abs(r).max()))
            log(f"  b{b} hk{hk} {name}: max err {err:.5f} scale {scale:.3f}")
            assert np.isfinite(x).all() and err <= TOL * scale

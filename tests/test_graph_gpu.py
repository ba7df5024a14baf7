"""The forward entry points inside a captured HIP graph.

The library only enqueues kernels on the caller's stream: it allocates nothing,
never synchronises and keeps no state, so a caller may record its launches in
a graph (bench.py times the forward steps that way). Each case captures one
call with preallocated outputs, replays the graph several times with unrelated
eager work and synchronisations in between, and checks every replay bit for bit
against the eager call (the kernels are deterministic).
"""

import pytest
import torch

import sdpa_inputs
from parity_util import log

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16", 128, True, (2, 8, 2, 300, 300)),
    ("bf16", 64, False, (2, 4, 4, 196, 196)),
    ("bf16", 64, True, (1, 4, 2, 1100, 1100)),  # the d = 64 ping-pong kernel (1024+ keys)
    ("fp8", 128, True, (1, 4, 1, 257, 257)),
    ("f32", 64, True, (1, 2, 2, 129, 129)),
]


def _eager_and_graph(call, outs, replays=3):
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for i in range(replays):
        for t in outs:
            t.fill_(float("nan"))
        junk.mul_(1.0001).add_(0.5)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t, r), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("dtype,d,causal,shape", CASES)
def test_forward_in_graph(gpu, dtype, d, causal, shape):
    import scaled_dot_product_18_amd as sdpa
    B, Hq, Hkv, Sq, Sk = shape
    w = sdpa_inputs.custom(B, Hq, Hkv, Sq, Sk, d, dtype, causal, seed=17000 + Sq + d)
    log(f"[graph] {w.name}")
    inp = sdpa_inputs.make_inputs(w)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    out_dtype = torch.float32 if dtype == "f32" else torch.bfloat16
    out = torch.empty((B, Hq, Sq, d), dtype=out_dtype, device="cuda")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    if dtype == "fp8":
        def call():
            sdpa.fwd_fp8(q, k, v, inp["descale_q"], inp["descale_k"], inp["descale_v"], causal=causal, scale=w.scale,
                         out=out, lse_out=lse)
    else:
        def call():
            sdpa.fwd(q, k, v, causal=causal, scale=w.scale, out=out, lse_out=lse)
    _eager_and_graph(call, [out, lse])


def test_splitkv_in_graph(gpu):
    import scaled_dot_product_18_amd as sdpa
    w = sdpa_inputs.custom(2, 8, 2, 1, 2000, 128, "bf16", False, seed=17500)
    log(f"[graph] {w.name} split-KV")
    inp = sdpa_inputs.make_inputs(w)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    splits, nbytes = sdpa.splitkv_plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.d)
    assert splits > 1
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.Hq, w.Sq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")

    def call():
        sdpa.fwd_splitkv(q, k, v, scale=w.scale, out=out, lse_out=lse, workspace=ws)
    _eager_and_graph(call, [out, lse])

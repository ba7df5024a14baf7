"""GPU parity of strided inputs and outputs (attn_fwd_strided): the codelab's own
(B, T, N, H) layout read and written in place, padded rows, and mixed layouts.

The kernels compute exactly what they compute on dense tensors, so besides the
oracle comparison at the dtype's tolerance every case also checks that the
strided result equals the dense one bit for bit.
"""

import itertools

import pytest
import torch

import sdpa_inputs
from parity_util import check_full, log, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _call(w, dev, q, k, v, **kw):
    import scaled_dot_product_18_amd as sdpa
    if w.dtype == "fp8":
        return sdpa.fwd_fp8(q, k, v, dev["descale_q"], dev["descale_k"], dev["descale_v"], causal=w.causal,
                            scale=w.scale, want_lse=True, **kw)
    return sdpa.fwd(q, k, v, causal=w.causal, scale=w.scale, want_lse=True, **kw)


@pytest.mark.parametrize("dtype,d,causal,S", list(itertools.product(("f32", "bf16", "fp8"), (64, 128), (False, True),
                                                                    (1, 65, 200))))
def test_codelab_layout_in_place(gpu, dtype, d, causal, S):
    """(B, T, N, H) tensors with layout="bshd": no permute, output in the same layout."""
    w = sdpa_inputs.custom(2, 4, 2, S, S, d, dtype, causal, seed=15000 + S + d, want_lse=True)
    log(f"[strided] {w.name} bshd")
    inp = sdpa_inputs.make_inputs(w)
    dev = to_device(inp)
    o_ref, lse_ref = run_gpu(w, dev)
    qs, ks, vs = (dev[n].transpose(1, 2).contiguous() for n in ("q", "k", "v"))  # (B, T, N, H) storage
    o, lse = _call(w, dev, qs, ks, vs, layout="bshd")
    torch.cuda.synchronize()
    assert o.shape == (w.B, w.Sq, w.Hq, w.d) and o.is_contiguous()
    o_bhsd = o.transpose(1, 2)
    check_full(w, inp, o_bhsd, lse)
    assert torch.equal(o_bhsd, o_ref) and torch.equal(lse, lse_ref)


@pytest.mark.parametrize("dtype,d,causal", list(itertools.product(("bf16", "fp8"), (32, 64), (False, True))))
def test_codelab_layout_key_split(gpu, dtype, d, causal):
    """bf16 and e4m3 at d = 32/64 with 700 keys on a small grid: the eight-wave key-split forms
    read and write (B, T, N, H) in place and equal their dense results bit for bit."""
    w = sdpa_inputs.custom(2, 4, 2, 700, 700, d, dtype, causal, seed=15500 + d, want_lse=True)
    log(f"[strided] {w.name} bshd split")
    inp = sdpa_inputs.make_inputs(w)
    dev = to_device(inp)
    o_ref, lse_ref = run_gpu(w, dev)
    qs, ks, vs = (dev[n].transpose(1, 2).contiguous() for n in ("q", "k", "v"))
    o, lse = _call(w, dev, qs, ks, vs, layout="bshd")
    torch.cuda.synchronize()
    o_bhsd = o.transpose(1, 2)
    check_full(w, inp, o_bhsd, lse)
    assert torch.equal(o_bhsd, o_ref) and torch.equal(lse, lse_ref)


@pytest.mark.parametrize("dtype,causal", list(itertools.product(("bf16", "fp8"), (False, True))))
def test_codelab_layout_ping_pong(gpu, dtype, causal):
    """bf16 and e4m3 at d = 64 with 1100 keys on a small grid: the eight-wave ping-pong kernel
    reads and writes (B, T, N, H) in place and equals its dense result bit for bit."""
    w = sdpa_inputs.custom(2, 4, 2, 1100, 1100, 64, dtype, causal, seed=15600, want_lse=True)
    log(f"[strided] {w.name} bshd ping-pong")
    inp = sdpa_inputs.make_inputs(w)
    dev = to_device(inp)
    o_ref, lse_ref = run_gpu(w, dev)
    qs, ks, vs = (dev[n].transpose(1, 2).contiguous() for n in ("q", "k", "v"))
    o, lse = _call(w, dev, qs, ks, vs, layout="bshd")
    torch.cuda.synchronize()
    o_bhsd = o.transpose(1, 2)
    check_full(w, inp, o_bhsd, lse)
    assert torch.equal(o_bhsd, o_ref) and torch.equal(lse, lse_ref)


@pytest.mark.parametrize("dtype,d", list(itertools.product(("f32", "bf16", "fp8"), (64, 128))))
def test_padded_rows_and_mixed_layouts(gpu, dtype, d):
    """q is every other row block of a wider tensor (position stride 2d), k and v are
    (B, T, N, H), the output is written into a slice of a larger buffer."""
    w = sdpa_inputs.custom(2, 4, 1, 77, 300, d, dtype, True, seed=16000 + d, want_lse=True)
    log(f"[strided] {w.name} mixed")
    inp = sdpa_inputs.make_inputs(w)
    dev = to_device(inp)
    o_ref, lse_ref = run_gpu(w, dev)
    wide = torch.zeros((w.B, w.Hq, w.Sq, 2 * d), dtype=dev["q"].dtype, device="cuda")
    wide[..., :d] = dev["q"]
    q = wide[..., :d]
    k = dev["k"].transpose(1, 2).contiguous().transpose(1, 2)
    v = dev["v"].transpose(1, 2).contiguous().transpose(1, 2)
    big = torch.full((w.B, w.Hq + 2, w.Sq, d), 7.0, dtype=o_ref.dtype, device="cuda")
    out = big[:, 1:w.Hq + 1]
    o, lse = _call(w, dev, q, k, v, out=out)
    torch.cuda.synchronize()
    check_full(w, inp, o, lse)
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    assert bool((big[:, 0] == 7.0).all()) and bool((big[:, -1] == 7.0).all())  # nothing written outside


def test_bad_strides_raise(gpu):
    import scaled_dot_product_18_amd as sdpa
    x = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        sdpa.fwd(x.transpose(2, 3), x, x)  # head dimension not contiguous
    odd = torch.zeros(1, 2, 16, 68, dtype=torch.bfloat16, device="cuda")[..., :64]  # 136-byte rows
    with pytest.raises(sdpa.AttnError) as e:
        sdpa.fwd(odd, x, x)
    assert e.value.status == -12

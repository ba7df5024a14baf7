"""Pins of the fp64 backward oracle (oracle.backward) to things other than itself.

  * central finite differences of the loss L = sum(O * dO) through the forward
    oracle (itself pinned in test_oracle.py): the definition of a derivative;
  * closed forms: a zero query makes every score equal, so dK = 0 and dV is the
    mean of dO (no mask); equal value rows make dQ = dK = 0; a single key has
    weight 1, so dV = sum of dO and dQ = dK = 0;
  * GQA: a KV head's gradient is the sum over the query heads that read it
    (MQA against MHA with the KV head repeated);
  * a library special case: torch's fp64 CPU attention differentiated by
    autograd (self-attention; its causal flag is the Sq == Sk mask).
Each pin takes the function under test as an argument, so a planted mistake in
a copy of the oracle is shown to fail at least one of them.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.backward import attention_backward


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float((o * do).sum())


def pin_finite_differences(bwd):
    rng = np.random.default_rng(11)
    for (B, Hq, Hkv, Sq, Sk, d), causal in [((1, 2, 1, 4, 6, 3), True), ((1, 2, 1, 4, 6, 3), False),
                                           ((2, 2, 2, 5, 5, 4), True), ((1, 3, 1, 3, 7, 2), False)]:
        q, k, v = _rand(rng, B, Hq, Sq, d), _rand(rng, B, Hkv, Sk, d), _rand(rng, B, Hkv, Sk, d)
        do = _rand(rng, B, Hq, Sq, d)
        scale = 0.7
        got = bwd(q, k, v, do, scale, causal)
        h = 1e-5
        for idx, x in enumerate((q, k, v)):
            fd = np.zeros_like(x)
            it = np.nditer(x, flags=["multi_index"])
            for _ in it:
                m = it.multi_index
                old = x[m]
                x[m] = old + h
                lp = _loss(q, k, v, do, scale, causal)
                x[m] = old - h
                lm = _loss(q, k, v, do, scale, causal)
                x[m] = old
                fd[m] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(got[idx], fd, atol=2e-7, rtol=0)


def pin_zero_query(bwd):
    rng = np.random.default_rng(12)
    B, Hq, Hkv, Sq, Sk, d = 1, 2, 2, 5, 7, 4
    q = np.zeros((B, Hq, Sq, d))
    k, v, do = _rand(rng, B, Hkv, Sk, d), _rand(rng, B, Hkv, Sk, d), _rand(rng, B, Hq, Sq, d)
    dq, dk, dv = bwd(q, k, v, do, 0.5, False)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv, np.broadcast_to(do.sum(axis=2, keepdims=True) / Sk, dv.shape), atol=1e-14)


def pin_equal_values(bwd):
    rng = np.random.default_rng(13)
    B, Hq, Hkv, Sq, Sk, d = 1, 2, 1, 6, 6, 3
    q, k, do = _rand(rng, B, Hq, Sq, d), _rand(rng, B, Hkv, Sk, d), _rand(rng, B, Hq, Sq, d)
    v = np.broadcast_to(_rand(rng, 1, 1, 1, d), (B, Hkv, Sk, d)).copy()
    for causal in (False, True):
        dq, dk, _ = bwd(q, k, v, do, 0.9, causal)
        np.testing.assert_allclose(dq, 0.0, atol=1e-13)
        np.testing.assert_allclose(dk, 0.0, atol=1e-13)


def pin_single_key(bwd):
    rng = np.random.default_rng(14)
    q, k, v, do = _rand(rng, 1, 3, 4, 5), _rand(rng, 1, 1, 1, 5), _rand(rng, 1, 1, 1, 5), _rand(rng, 1, 3, 4, 5)
    dq, dk, dv = bwd(q, k, v, do, 0.3, False)
    np.testing.assert_allclose(dq, 0.0, atol=1e-14)
    np.testing.assert_allclose(dk, 0.0, atol=1e-14)
    np.testing.assert_allclose(dv[0, 0, 0], do.sum(axis=(0, 1, 2)), atol=1e-13)


def pin_gqa_is_mha_sum(bwd):
    rng = np.random.default_rng(15)
    B, Hq, Sq, Sk, d = 2, 4, 5, 8, 3
    q, do = _rand(rng, B, Hq, Sq, d), _rand(rng, B, Hq, Sq, d)
    k1, v1 = _rand(rng, B, 2, Sk, d), _rand(rng, B, 2, Sk, d)
    for causal in (False, True):
        dq_g, dk_g, dv_g = bwd(q, k1, v1, do, 0.6, causal)
        kr, vr = np.repeat(k1, 2, axis=1), np.repeat(v1, 2, axis=1)  # query head h reads KV head h // 2
        dq_m, dk_m, dv_m = bwd(q, kr, vr, do, 0.6, causal)
        np.testing.assert_allclose(dq_g, dq_m, atol=1e-13)
        np.testing.assert_allclose(dk_g, dk_m.reshape(B, 2, 2, Sk, d).sum(axis=2), atol=1e-13)
        np.testing.assert_allclose(dv_g, dv_m.reshape(B, 2, 2, Sk, d).sum(axis=2), atol=1e-13)


def pin_torch_autograd(bwd):
    rng = np.random.default_rng(16)
    B, H, S, d = 2, 3, 9, 5
    q, k, v, do = (_rand(rng, B, H, S, d) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.4)
        o.backward(torch.tensor(do))
        got = bwd(q, k, v, do, 0.4, causal)
        for g, t in zip(got, (tq, tk, tv)):
            np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12)


PINS = [pin_finite_differences, pin_zero_query, pin_equal_values, pin_single_key, pin_gqa_is_mha_sum,
        pin_torch_autograd]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(attention_backward)


def test_backward_rejects_bad_shapes():
    z = np.zeros((1, 2, 3, 4))
    with pytest.raises(ValueError):
        attention_backward(z, z, z, np.zeros((1, 2, 3, 5)), 1.0)
    with pytest.raises(ValueError):
        attention_backward(np.zeros((1, 2, 5, 4)), z, z, np.zeros((1, 2, 5, 4)), 1.0, causal=True)


# ------------------------------------------------------------- planted mistakes

def _mutant(kind):
    def bwd(q, k, v, do, scale, causal):
        B, Hq, Sq, d = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        G = Hq // Hkv
        dq = np.zeros(q.shape)
        dk = np.zeros(k.shape)
        dv = np.zeros(v.shape)
        for b in range(B):
            for h in range(Hq):
                hk = (h % Hkv) if kind == "head_modulo" else h // G
                s = (q[b, h] @ k[b, hk].T) * scale
                if causal:
                    off = 1 if kind == "causal_off_by_one" else 0
                    keep = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] + Sk - Sq + off
                    s = np.where(keep, s, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                g = do[b, h]
                dp = g @ v[b, hk].T
                if kind == "no_jacobian_term":
                    ds = p * dp
                elif kind == "jacobian_sign":
                    ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))
                else:
                    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dv[b, hk] += (ds.T if kind == "dv_from_ds" else p.T) @ g
                sq = 1.0 if kind == "dq_unscaled" else scale
                dq[b, h] = sq * (ds @ (v[b, hk] if kind == "dq_uses_v" else k[b, hk]))
                dk[b, hk] += (1.0 if kind == "dk_unscaled" else scale) * (ds.T @ q[b, h])
        return dq, dk, dv
    return bwd


MUTANTS = ["no_jacobian_term", "jacobian_sign", "dv_from_ds", "dq_unscaled", "dq_uses_v", "dk_unscaled",
           "head_modulo", "causal_off_by_one"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    caught = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin(_mutant(kind))
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {kind!r}"


def test_unmutated_copy_passes_every_pin():
    for pin in PINS:
        pin(_mutant("none"))

"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each pin is a function of an attention callable with the oracle's signature
``attn(q, k, v, scale, causal) -> (O, lse)``, so the same checks run against
the oracle (must pass) and against planted mistakes (each must fail at least
one pin): a dropped scale, a flipped sign, swapped K/V, a wrong KV-head
mapping, an off-by-one causal mask, log2 statistics, a missing max
subtraction, a transposed value contraction.
"""

import math
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3
from golden_io import load_all

RNG = np.random.default_rng(1234)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# --------------------------------------------------------------------------- pins

def pin_golden(attn):
    """Hand-derived fixtures (tests/golden/*.json, each citing the pages)."""
    for c in load_all():
        o, lse = attn(c["q"], c["k"], c["v"], c["scale"], c["causal"])
        np.testing.assert_allclose(o, c["o"], rtol=0, atol=1e-13, err_msg=c["name"])
        np.testing.assert_allclose(lse, c["lse"], rtol=0, atol=1e-13, err_msg=c["name"])


def pin_single_key(attn):
    """One key: the weight is 1, so O = V[0] and lse is the one scaled score."""
    q, k, v = _rand(2, 3, 5, 16), _rand(2, 3, 1, 16), _rand(2, 3, 1, 16)
    o, lse = attn(q, k, v, 0.3, False)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, 0.3 * np.einsum("bhid,bhjd->bhi", q, k), atol=1e-13)


def pin_rows_sum_to_one(attn):
    """With V the identity (d = Sk) the output rows ARE the weights: >= 0, rows sum to 1,
    and under the causal mask every weight above the diagonal is 0."""
    S = 24
    q, k = _rand(1, 2, S, S), _rand(1, 2, S, S)
    v = np.broadcast_to(np.eye(S), (1, 2, S, S)).copy()
    for causal in (False, True):
        w, _ = attn(q, k, v, 1.0 / math.sqrt(S), causal)
        assert np.all(w >= 0)
        np.testing.assert_allclose(w.sum(-1), 1.0, atol=1e-13)
        if causal:
            assert np.all(np.triu(w[0, 0], 1) == 0) and np.all(np.triu(w[0, 1], 1) == 0)
            np.testing.assert_allclose(w[0, :, 0, 0], 1.0, atol=0)


def pin_equal_keys_mean(attn):
    """All keys equal: uniform weights, so O is the mean of the allowed V rows."""
    S, d = 13, 8
    q = _rand(1, 1, S, d)
    k = np.broadcast_to(_rand(1, 1, 1, d), (1, 1, S, d)).copy()
    v = _rand(1, 1, S, d)
    o, lse = attn(q, k, v, 0.7, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(0), (S, d)), atol=1e-13)
    oc, _ = attn(q, k, v, 0.7, True)
    cummean = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(oc[0, 0], cummean, atol=1e-13)


def pin_causal_first_last(attn):
    """Causal row 0 attends only to itself; the causal last row equals the unmasked one."""
    S, d = 17, 8
    q, k, v = _rand(2, 2, S, d), _rand(2, 2, S, d), _rand(2, 2, S, d)
    oc, lc = attn(q, k, v, 0.25, True)
    on, ln_ = attn(q, k, v, 0.25, False)
    np.testing.assert_allclose(oc[:, :, 0], v[:, :, 0], atol=1e-14)
    np.testing.assert_allclose(lc[:, :, 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-13)
    np.testing.assert_allclose(oc[:, :, -1], on[:, :, -1], atol=1e-13)
    np.testing.assert_allclose(lc[:, :, -1], ln_[:, :, -1], atol=1e-13)
    assert np.max(np.abs(oc[:, :, 0] - on[:, :, 0])) > 1e-3


def pin_gqa_is_repeated_mha(attn):
    """GQA/MQA equal MHA with each KV head repeated over its group of query heads."""
    B, Hq, S, d = 2, 8, 9, 8
    q = _rand(B, Hq, S, d)
    for Hkv in (8, 2, 1):
        k, v = _rand(B, Hkv, S, d), _rand(B, Hkv, S, d)
        G = Hq // Hkv
        o, lse = attn(q, k, v, 0.35, False)
        o_ref, lse_ref = attn(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.35, False)
        np.testing.assert_allclose(o, o_ref, atol=1e-14)
        np.testing.assert_allclose(lse, lse_ref, atol=1e-13)
        # independent: torch's grouped routine on the same values
        t = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.35, enable_gqa=True)
        np.testing.assert_allclose(o, t.numpy(), atol=1e-12)


def pin_shift_affine_permutation(attn):
    """Adding c to every key leaves O unchanged and moves lse by scale*q.c;
    V -> aV + b maps O -> aO + b; permuting keys (unmasked) leaves O unchanged."""
    S, d, sc = 11, 8, 0.4
    q, k, v = _rand(1, 2, S, d), _rand(1, 2, S, d), _rand(1, 2, S, d)
    o, lse = attn(q, k, v, sc, False)
    c = _rand(d)
    o2, lse2 = attn(q, k + c, v, sc, False)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2 - sc * (q @ c), lse, atol=1e-12)
    oc, _ = attn(q, k, v, sc, True)
    oc2, _ = attn(q, k + c, v, sc, True)
    np.testing.assert_allclose(oc2, oc, atol=1e-13)
    o3, _ = attn(q, k, 2.5 * v - 1.25, sc, False)
    np.testing.assert_allclose(o3, 2.5 * o - 1.25, atol=1e-12)
    perm = RNG.permutation(S)
    o4, lse4 = attn(q, k[:, :, perm], v[:, :, perm], sc, False)
    np.testing.assert_allclose(o4, o, atol=1e-13)
    np.testing.assert_allclose(lse4, lse, atol=1e-13)


def pin_large_offset(attn):
    """Scores near 1e3: the definition is still finite (max subtraction)."""
    S, d = 6, 4
    q = np.full((1, 1, S, d), 30.0)
    k = np.full((1, 1, S, d), 30.0) + _rand(1, 1, S, d) * 0.1
    v = _rand(1, 1, S, d)
    o, lse = attn(q, k, v, 0.25, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.all(lse > 800)


def _decimal_attention(q, k, v, scale, causal):
    getcontext().prec = 50
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Hq, Sq, d))
    lse = np.zeros((B, Hq, Sq))
    D = Decimal
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            for i in range(Sq):
                js = [j for j in range(Sk) if (not causal) or j <= i + Sk - Sq]
                s = [D(scale) * sum(D(q[b, h, i, c]) * D(k[b, hk, j, c]) for c in range(d)) for j in js]
                e = [x.exp() for x in s]
                den = sum(e)
                for c in range(d):
                    o[b, h, i, c] = float(sum(e[t] * D(v[b, hk, j, c]) for t, j in enumerate(js)) / den)
                lse[b, h, i] = float(den.ln())
    return o, lse


def pin_decimal_bruteforce(attn):
    """50-digit Decimal evaluation of the definition on tiny inputs (S <= 5, d <= 4), including
    queries that are the last Sq of Sk positions."""
    for (B, Hq, Hkv, Sq, Sk, d, causal, sc) in [(1, 1, 1, 4, 4, 4, False, 0.5), (1, 2, 1, 4, 4, 3, True, 0.9),
                                                (2, 4, 2, 3, 3, 2, False, 1.3), (1, 2, 2, 1, 1, 4, True, 0.5),
                                                (1, 1, 1, 4, 4, 1, True, 2.0), (1, 2, 1, 2, 5, 3, True, 0.8),
                                                (1, 1, 1, 3, 5, 2, False, 1.1)]:
        q, k, v = _rand(B, Hq, Sq, d, scale=1.5), _rand(B, Hkv, Sk, d, scale=1.5), _rand(B, Hkv, Sk, d)
        o, lse = attn(q, k, v, sc, causal)
        o_ref, lse_ref = _decimal_attention(q, k, v, sc, causal)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-14)


def pin_torch_library(attn):
    """torch's fp64 CPU attention (a library routine independent of this oracle), with
    its causal flag, its grouped-query option, and its log-sum-exp output."""
    for (B, Hq, Hkv, S, d, causal) in [(2, 4, 4, 33, 16, False), (1, 8, 2, 40, 32, True), (2, 4, 1, 19, 8, True)]:
        q, k, v = _rand(B, Hq, S, d), _rand(B, Hkv, S, d), _rand(B, Hkv, S, d)
        sc = 1.0 / math.sqrt(d)
        o, lse = attn(q, k, v, sc, causal)
        G = Hq // Hkv
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(np.repeat(k, G, axis=1))
        tv = torch.from_numpy(np.repeat(v, G, axis=1))
        to, tlse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(tq, tk, tv, 0.0, causal, scale=sc)[:2]
        np.testing.assert_allclose(o, to.numpy(), atol=1e-12)
        np.testing.assert_allclose(lse, tlse.numpy(), atol=1e-12)


def pin_queries_at_the_end(attn):
    """Causal Sq < Sk: the queries are the last Sq positions. Their rows equal the last Sq rows of
    the square causal problem whose earlier query rows are arbitrary; the last row sees every key,
    so it equals the unmasked row; a single query (decode) is unmasked."""
    B, Hq, Hkv, Sq, Sk, d, sc = 2, 4, 2, 5, 19, 8, 0.45
    q, k, v = _rand(B, Hq, Sq, d), _rand(B, Hkv, Sk, d), _rand(B, Hkv, Sk, d)
    o, lse = attn(q, k, v, sc, True)
    q_full = np.concatenate([_rand(B, Hq, Sk - Sq, d), q], axis=2)
    of, lf = attn(q_full, k, v, sc, True)
    np.testing.assert_allclose(o, of[:, :, Sk - Sq:], atol=1e-13)
    np.testing.assert_allclose(lse, lf[:, :, Sk - Sq:], atol=1e-13)
    on, ln_ = attn(q, k, v, sc, False)
    np.testing.assert_allclose(o[:, :, -1], on[:, :, -1], atol=1e-13)
    assert np.max(np.abs(o[:, :, 0] - on[:, :, 0])) > 1e-3
    o1, l1 = attn(q[:, :, -1:], k, v, sc, True)
    np.testing.assert_allclose(o1, on[:, :, -1:], atol=1e-13)
    np.testing.assert_allclose(l1, ln_[:, :, -1:], atol=1e-13)


def pin_split_keys_merge(attn):
    """Attention over two disjoint key sets combines through the row statistic: with
    lse = ln(exp lse1 + exp lse2), O = exp(lse1 - lse) O1 + exp(lse2 - lse) O2."""
    B, Hq, Hkv, Sq, Sk, d, sc = 1, 4, 1, 3, 23, 8, 0.6
    q, k, v = _rand(B, Hq, Sq, d), _rand(B, Hkv, Sk, d, scale=2.0), _rand(B, Hkv, Sk, d)
    o, lse = attn(q, k, v, sc, False)
    c = 9
    o1, l1 = attn(q, k[:, :, :c], v[:, :, :c], sc, False)
    o2, l2 = attn(q, k[:, :, c:], v[:, :, c:], sc, False)
    lm = np.logaddexp(l1, l2)
    np.testing.assert_allclose(lm, lse, atol=1e-13)
    np.testing.assert_allclose(np.exp(l1 - lm)[..., None] * o1 + np.exp(l2 - lm)[..., None] * o2, o, atol=1e-13)


PINS = [pin_golden, pin_single_key, pin_rows_sum_to_one, pin_equal_keys_mean, pin_causal_first_last,
        pin_gqa_is_repeated_mha, pin_shift_affine_permutation, pin_large_offset, pin_decimal_bruteforce,
        pin_torch_library, pin_queries_at_the_end, pin_split_keys_merge]


def _oracle(q, k, v, scale, causal):
    return oracle.attention(q, k, v, scale, causal)


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(_oracle)


def test_sampled_rows_match_full():
    q, k, v = _rand(2, 4, 37, 8), _rand(2, 2, 37, 8), _rand(2, 2, 37, 8)
    o, lse = oracle.attention(q, k, v, 0.3, True, row_block=7)
    rows = np.array([0, 5, 36, 18])
    for b, h, r, os_, ls in oracle.attention_sampled(q, k, v, 0.3, True, [(1, 3, rows), (0, 0, rows)]):
        np.testing.assert_array_equal(os_, o[b, h, r])
        np.testing.assert_array_equal(ls, lse[b, h, r])


def test_oracle_rejects_bad_shapes():
    q, k = np.zeros((1, 3, 4, 8)), np.zeros((1, 2, 4, 8))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, 1.0)
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 2, 5, 8)), k, k, 1.0, causal=True)
    oracle.attention(np.zeros((1, 2, 3, 8)), k, k, 1.0, causal=True)


# --------------------------------------------------------------------- E4M3 decoder

def test_e4m3_decoder_exhaustive_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x38] == 1.0


# ------------------------------------------------------------- planted mistakes

def _mutant(kind):
    def attn(q, k, v, scale, causal):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, Hq, Sq, d = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        G = Hq // Hkv
        o = np.zeros((B, Hq, Sq, v.shape[3]))
        lse = np.zeros((B, Hq, Sq))
        for b in range(B):
            for h in range(Hq):
                hk = (h % Hkv) if kind == "head_modulo" else h // G
                kk, vv = (v[b, hk], k[b, hk]) if kind == "swap_kv" else (k[b, hk], v[b, hk])
                sc = 1.0 if kind == "no_scale" else scale
                s = (q[b, h] @ kk.T) * sc
                if kind == "neg_sign":
                    s = -s
                if causal:
                    i = np.arange(Sq)[:, None]
                    j = np.arange(Sk)[None, :]
                    off = 0 if kind == "top_left" else Sk - Sq
                    keep = (j <= i + off + 1) if kind == "causal_off_by_one" else (j <= i + off)
                    s = np.where(keep, s, -np.inf)
                if kind == "no_max":
                    e = np.exp(s)
                    m = np.zeros((Sq, 1))
                else:
                    m = s.max(axis=1, keepdims=True)
                    e = np.exp(s - m)
                den = e.sum(axis=1, keepdims=True)
                w = e / den
                o[b, h] = (w.T @ vv if (kind == "transpose_w" and Sq == Sk) else w @ vv)
                lse[b, h] = (m[:, 0] + np.log2(den[:, 0])) if kind == "lse_log2" else (m[:, 0] + np.log(den[:, 0]))
        return o, lse
    return attn


MUTANTS = ["no_scale", "neg_sign", "swap_kv", "head_modulo", "causal_off_by_one", "lse_log2", "no_max",
           "transpose_w", "top_left"]


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
    """The mutant scaffold itself is faithful, so the failures above come from the planted mistakes."""
    for pin in PINS:
        pin(_mutant("none"))

"""Pins of the seeded input generator and of the fp8 dequantiser (CPU only).

The generator feeds both the HIP path and the oracle, so a mistake in it would
move both sides at once and parity would not notice. These tests tie it to
facts outside itself:
  * determinism: a seed gives the same bytes every time, other seeds differ;
  * the GQA/MQA workloads share their queries (codelab "Accelerate attention on
    GPU with cuDNN and TransformerEngine", section 9, draws one Q for the MHA,
    GQA and MQA cells) while K and V are drawn per KV-head count;
  * the draws are standard normal (the codelab's input cells);
  * bf16 inputs are the round-to-nearest-even cast of the fp32 draws, checked
    against bit arithmetic on the fp32 words;
  * the per-tensor amax E4M3 quantiser (section 10) maps amax to 448, its
    descale is amax / 448 in fp32, and its codes equal a brute-force nearest
    value search over the decoder's table with ties to the even code;
  * the oracle's dequantiser returns code value times descale: the amax
    element comes back as amax, and every element within half an E4M3 step;
  * the same for the E5M2 gradient format of the fp8 backward pass (section
    10): the decoder exhaustively against torch.float8_e5m2, the amax
    quantiser against a brute-force nearest-even search, the round trip.
"""

import math

import numpy as np
import pytest
import torch

import sdpa_inputs
from oracle import e4m3


# ----------------------------------------------------------------- determinism

def test_same_seed_same_bytes():
    for dtype in ("f32", "bf16", "fp8"):
        w = sdpa_inputs.custom(2, 4, 2, 33, 40, 64, dtype, True, seed=123)
        a, b = sdpa_inputs.make_inputs(w), sdpa_inputs.make_inputs(w)
        for n in ("q", "k", "v"):
            assert a[n].dtype == b[n].dtype
            assert torch.equal(a[n].view(torch.uint8) if a[n].dtype != torch.uint8 else a[n],
                               b[n].view(torch.uint8) if b[n].dtype != torch.uint8 else b[n])
        assert a["descale_q"] == b["descale_q"] and a["descale_v"] == b["descale_v"]
        c = sdpa_inputs.make_inputs(w, seed=124)
        for n in ("q", "k", "v"):
            assert not torch.equal(a[n], c[n])


def test_streams_of_q_k_v_are_distinct():
    w = sdpa_inputs.custom(1, 2, 2, 16, 16, 64, "f32", False, seed=5)
    inp = sdpa_inputs.make_inputs(w)
    assert not torch.equal(inp["q"], inp["k"]) and not torch.equal(inp["k"], inp["v"])


def test_queries_shared_across_kv_head_counts():
    """Same seed and query shape, Hkv = 8, 2, 1: one Q, different K and V."""
    ins = [sdpa_inputs.make_inputs(sdpa_inputs.custom(2, 8, hkv, 64, 64, 64, "bf16", True, seed=42))
           for hkv in (8, 2, 1)]
    assert torch.equal(ins[0]["q"], ins[1]["q"]) and torch.equal(ins[0]["q"], ins[2]["q"])
    assert ins[0]["k"].shape[1] == 8 and ins[2]["k"].shape[1] == 1
    assert not torch.equal(ins[1]["k"][:, :1], ins[2]["k"])


def test_headline_workloads_share_queries():
    gqa = sdpa_inputs.WORKLOADS["causal_gqa_bf16_b4_hq32_hkv8_s4096_d128"]
    mqa = sdpa_inputs.WORKLOADS["causal_mqa_bf16_b4_hq32_hkv1_s4096_d128"]
    assert (gqa.seed, gqa.B, gqa.Hq, gqa.Sq, gqa.d) == (mqa.seed, mqa.B, mqa.Hq, mqa.Sq, mqa.d)
    # the query stream depends on (seed, shape of Q) only: a slice of both draws agrees
    q1, _, _ = sdpa_inputs.draw_qkv(1, 2, 2, 8, 8, 16, gqa.seed)
    q2, _, _ = sdpa_inputs.draw_qkv(1, 2, 1, 8, 8, 16, mqa.seed)
    assert torch.equal(q1, q2)


# ------------------------------------------------------------ distribution

def test_draws_are_standard_normal():
    q, k, v = sdpa_inputs.draw_qkv(4, 8, 8, 256, 256, 64, seed=0)
    for t in (q, k, v):
        x = t.double().numpy().ravel()
        n = x.size  # 524288 draws: the sample mean has sd 1/sqrt(n) = 1.4e-3
        assert abs(x.mean()) < 6 / math.sqrt(n)
        assert abs(x.std() - 1.0) < 6 * math.sqrt(0.5 / n)
        # fraction within one standard deviation: 0.6827 for N(0, 1)
        assert abs(np.mean(np.abs(x) < 1.0) - 0.682689) < 0.005


def _bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values, round to nearest even, from the fp32 words."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_bf16_inputs_are_rne_of_the_fp32_draws():
    w32 = sdpa_inputs.custom(2, 4, 2, 100, 100, 64, "f32", False, seed=77)
    w16 = sdpa_inputs.custom(2, 4, 2, 100, 100, 64, "bf16", False, seed=77)
    a, b = sdpa_inputs.make_inputs(w32), sdpa_inputs.make_inputs(w16)
    for n in ("q", "k", "v"):
        want = _bf16_rne_bits(a[n].numpy())
        got = b[n].view(torch.int16).numpy().view(np.uint16)
        np.testing.assert_array_equal(got, want)


# -------------------------------------------------------------- e4m3 quantiser

def _finite_table():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3.decode(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]


def _encode_brute_force(y: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3fn value to each y (|y| <= 448), ties to the code with an
    even mantissa; +0 for values that round to zero from either side."""
    codes, vals = _finite_table()
    y = np.asarray(y, dtype=np.float64)
    out = np.empty(y.shape, dtype=np.uint8)
    for idx, x in np.ndenumerate(y):
        dist = np.abs(vals - x)
        best = dist.min()
        cand = codes[dist == best]
        if len(cand) > 1:
            # a tie between two neighbours (or between +0 and -0): take the even mantissa,
            # and the sign of x for a zero
            nz = [c for c in cand if e4m3.decode_code(c) != 0.0]
            if nz:
                even = [c for c in cand if (c & 1) == 0]
                cand = even if even else cand
            else:
                cand = [0x80 if math.copysign(1.0, x) < 0 else 0x00]
        out[idx] = cand[0]
    return out


def test_quantiser_matches_brute_force_nearest_even():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4000, generator=g, dtype=torch.float32) * 3.0
    codes, descale = sdpa_inputs.quantise_e4m3(x)
    s = np.float32(448.0) / np.float32(float(x.abs().max()))
    y = np.clip(x.numpy() * s, -448.0, 448.0)  # fp32 product, as the quantiser forms it
    np.testing.assert_array_equal(codes.numpy(), _encode_brute_force(y))


def test_quantiser_ties_go_to_even_and_saturate_at_448():
    # amax 448 gives a scale of exactly 1, so these values reach the rounding unchanged
    ties = [1.0625, 1.1875, 1.3125, 17.0, 19.0, 3.0 * 2.0 ** -10, 2.0 ** -10, 416.0, 432.0, -1.0625, -432.0]
    x = torch.tensor(ties + [448.0, -448.0, 447.0, 2.0 ** -12], dtype=torch.float32)
    codes, descale = sdpa_inputs.quantise_e4m3(x)
    assert descale == 1.0
    got = e4m3.decode(codes.numpy())
    want = [1.0, 1.25, 1.25, 16.0, 20.0, 2.0 ** -8, 0.0, 416.0, 448.0, -1.0, -448.0, 448.0, -448.0, 448.0, 0.0]
    np.testing.assert_array_equal(got, np.array(want))
    np.testing.assert_array_equal(codes.numpy(), _encode_brute_force(x.numpy()))


@pytest.mark.parametrize("amax", [1e-3, 0.37, 4.0, 5000.0])
def test_quantiser_amax_maps_to_448_and_descale_is_amax_over_448(amax):
    g = torch.Generator().manual_seed(int(amax * 1000) % 997)
    x = torch.rand(999, generator=g, dtype=torch.float32) * 2 - 1
    x = x / x.abs().max() * amax
    i = int(x.abs().argmax())
    codes, descale = sdpa_inputs.quantise_e4m3(x)
    assert abs(e4m3.decode(codes.numpy()[i:i + 1])[0]) == 448.0
    a32 = np.float32(float(x.abs().max()))
    assert descale == float(np.float32(1.0) / (np.float32(448.0) / a32))
    assert abs(descale - float(a32) / 448.0) <= 2 * np.spacing(np.float32(descale))


# ---------------------------------------------------------------- dequantiser

@pytest.mark.parametrize("amax", [1e-2, 1.0, 4.7, 300.0])
def test_dequantise_round_trips_within_half_a_step(amax):
    g = torch.Generator().manual_seed(11)
    x = torch.randn(5000, generator=g, dtype=torch.float32)
    x = x / x.abs().max() * amax
    codes, descale = sdpa_inputs.quantise_e4m3(x)
    back = e4m3.dequantise(codes.numpy(), descale)
    xs = x.double().numpy()
    # the amax element comes back as amax (448 * descale; descale carries fp32 rounding)
    i = int(np.abs(xs).argmax())
    assert abs(abs(back[i]) - amax) <= 4 * 2.0 ** -24 * amax
    assert np.sign(back[i]) == np.sign(xs[i])
    # every element within half an E4M3 step of its scaled value: 2^(e - 4) for
    # |x s| in [2^e, 2^(e+1)) with e >= -6, 2^-10 in the subnormal range
    y = np.abs(xs) / descale
    step_half = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 4), 2.0 ** -10)
    assert np.all(np.abs(back - xs) <= (step_half * (1 + 1e-6) + 1e-7 * y) * descale)


def test_dequantise_is_code_value_times_descale():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3.decode(codes)
    ok = ~np.isnan(vals)
    np.testing.assert_array_equal(e4m3.dequantise(codes, None)[ok], vals[ok])
    np.testing.assert_array_equal(e4m3.dequantise(codes, 1.0)[ok], vals[ok])
    d = float(np.float32(0.0123))
    got = e4m3.dequantise(codes, d)[ok]
    # exact in fp64: a 4-bit significand times a 24-bit one
    np.testing.assert_array_equal(got, vals[ok] * d)
    assert e4m3.dequantise(np.array([0x7E], dtype=np.uint8), d)[0] == 448.0 * d
    assert e4m3.dequantise(np.array([0x01], dtype=np.uint8), 2.0)[0] == 2.0 ** -8


# ------------------------------------------------------- e5m2 (fp8 gradients)

def test_e5m2_decoder_exhaustive_against_torch():
    from oracle import e5m2
    codes = np.arange(256, dtype=np.uint8)
    ours = e5m2.decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF]
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert ours[0x7B] == 57344.0 and ours[0x7C] == np.inf and ours[0xFC] == -np.inf
    assert ours[0x01] == 2.0 ** -16 and ours[0x04] == 2.0 ** -14 and ours[0x3C] == 1.0


def _e5m2_encode_brute_force(y):
    """Nearest finite E5M2 value (|y| <= 57344), ties to the even mantissa."""
    from oracle import e5m2
    codes = np.arange(256, dtype=np.uint8)
    vals = e5m2.decode(codes)
    keep = np.isfinite(vals)
    codes, vals = codes[keep], vals[keep]
    out = np.empty(np.shape(y), dtype=np.uint8)
    for idx, x in np.ndenumerate(np.asarray(y, dtype=np.float64)):
        dist = np.abs(vals - x)
        cand = codes[dist == dist.min()]
        if len(cand) > 1:
            nz = [c for c in cand if e5m2.decode_code(c) != 0.0]
            if nz:
                cand = [c for c in cand if (c & 1) == 0] or list(cand)
            else:
                cand = [0x80 if math.copysign(1.0, x) < 0 else 0x00]
        out[idx] = cand[0]
    return out


def test_e5m2_quantiser_matches_brute_force_and_saturates():
    g = torch.Generator().manual_seed(8)
    x = torch.randn(3000, generator=g, dtype=torch.float32) * 0.3
    codes, descale = sdpa_inputs.quantise_e5m2(x)
    s = np.float32(sdpa_inputs.E5M2_MAX) / np.float32(float(x.abs().max()))
    y = np.clip(x.numpy() * s, -57344.0, 57344.0)
    np.testing.assert_array_equal(codes.numpy(), _e5m2_encode_brute_force(y))
    # amax 57344 gives a scale of exactly 1: ties go to the even mantissa (53248 lies halfway between
    # 49152 and 57344), and the largest finite value stays
    t = torch.tensor([1.125, 1.375, 3.5 * 2.0 ** -16, 2.0 ** -17, 53248.0, 57344.0, -1.125, 2.0 ** -18],
                     dtype=torch.float32)
    codes, descale = sdpa_inputs.quantise_e5m2(t)
    assert descale == 1.0
    from oracle import e5m2
    np.testing.assert_array_equal(e5m2.decode(codes.numpy()),
                                  [1.0, 1.5, 2.0 ** -14, 0.0, 49152.0, 57344.0, -1.0, 0.0])


def test_e5m2_dequantise_round_trips_within_half_a_step():
    from oracle import e5m2
    g = torch.Generator().manual_seed(12)
    x = torch.randn(5000, generator=g, dtype=torch.float32) * 0.05
    codes, descale = sdpa_inputs.quantise_e5m2(x)
    back = e5m2.dequantise(codes.numpy(), descale)
    xs = x.double().numpy()
    i = int(np.abs(xs).argmax())
    assert abs(abs(back[i]) - np.abs(xs).max()) <= 4 * 2.0 ** -24 * np.abs(xs).max()
    y = np.abs(xs) / descale
    # half a step: 2^(e - 3) for |x s| in [2^e, 2^(e+1)), e >= -14; 2^-17 below
    step_half = np.where(y >= 2.0 ** -14, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -14))) - 3), 2.0 ** -17)
    assert np.all(np.abs(back - xs) <= (step_half * (1 + 1e-6) + 1e-7 * y) * descale)
    assert e5m2.dequantise(np.array([0x3C], dtype=np.uint8), 0.5)[0] == 0.5


def test_fp8_gradient_draw_is_the_bf16_gradient_stream():
    w = sdpa_inputs.custom(1, 2, 1, 40, 40, 64, "fp8", True, seed=77)
    codes, descale = sdpa_inputs.draw_grad_fp8(w)
    ref = sdpa_inputs.draw_grad(w).float()  # same N(0,1) stream, rounded to bf16
    from oracle import e5m2
    back = torch.from_numpy(e5m2.dequantise(codes.numpy(), descale)).float()
    assert codes.shape == (1, 2, 40, 64) and codes.dtype == torch.uint8
    assert float((back - ref).abs().max()) <= 0.13 * float(ref.abs().max())

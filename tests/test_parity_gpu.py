"""GPU parity of the fused HIP kernels against the fp64 oracle, through the C ABI.

Small problems (spanning several tiles and a ragged tail) are compared element
by element with the full oracle; the full-size workloads are launched exactly
as the benchmark launches them and compared on sampled rows, which the oracle
computes one by one. Tolerances are max |GPU - oracle|: 1e-4 fp32, 2e-2 bf16,
6e-2 fp8 (on dequantised inputs), the fp8 rows whose P.V takes P rounded to
e4m3 (d = 128, rows that see 256 keys or more) plus a per-element bound
derived from the exact softmax weights (parity_util.p8_bound); lse 1e-4 for
fp32 and bf16, 1e-3 for fp8 (parity_util derives the bounds).
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs
from golden_io import load_all
from parity_util import TOL_LSE, TOL_O, check_full, check_sampled, log, run_gpu, to_device

pytestmark = pytest.mark.gpu

TAIL_S = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 196, 255, 257]
HEADS = [(8, 8), (8, 4), (8, 2), (8, 1)]


def _run_full(w, want_lse=True):
    log(f"[parity] {w.name}")
    inp = sdpa_inputs.make_inputs(w)
    o, lse = run_gpu(w, to_device(inp), want_lse=want_lse)
    torch.cuda.synchronize()
    return check_full(w, inp, o, lse)


# ------------------------------------------------------------ the small workloads

def test_single_head_f32_workload(gpu):
    stats = _run_full(sdpa_inputs.WORKLOADS["single_head_f32_s128_d64"])
    log(f"  {stats}")


def test_vit_b16_bf16_workload(gpu):
    stats = _run_full(sdpa_inputs.WORKLOADS["vit_b16_bf16_b32_h12_s196_d64"])
    log(f"  {stats}")


# ------------------------------------------------------- tails, heads, causal

@pytest.mark.parametrize("S,d,causal,heads", list(itertools.product(TAIL_S, (32, 64, 128), (False, True), HEADS)))
def test_bf16_tails(gpu, S, d, causal, heads):
    Hq, Hkv = heads
    w = sdpa_inputs.custom(1, Hq, Hkv, S, S, d, "bf16", causal, seed=1000 + S)
    _run_full(w)


# bf16 at d = 32 and 64: grids of at most 256 workgroups with at least 384
# keys split each workgroup's keys over eight waves (two halves of the key
# tiles, merged at the end); other grids up to 768 workgroups read operands
# ahead with four waves; larger grids take the plain four-wave form. Odd and
# even tile counts, the 383/384-key and 256/264-workgroup boundaries, causal
# rows whose second half sees no key (Sq < Sk), ragged tails, GQA and MQA.
SMALL_D_FORMS = [
    (1, 4, 2, 384, 384, 64, False), (1, 4, 2, 383, 383, 64, True), (1, 4, 4, 449, 449, 64, True),
    (2, 4, 1, 700, 700, 64, False), (1, 8, 2, 130, 1000, 64, True), (2, 4, 2, 5, 1000, 64, True),
    (1, 8, 8, 1024, 1024, 32, True), (1, 4, 2, 77, 640, 32, False), (1, 32, 8, 1024, 1024, 64, True),
    (1, 33, 11, 1024, 1024, 64, False), (4, 12, 4, 520, 520, 64, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,causal", SMALL_D_FORMS)
def test_bf16_small_head_dim_forms(gpu, B, Hq, Hkv, Sq, Sk, d, causal):
    stats = _run_full(sdpa_inputs.custom(B, Hq, Hkv, Sq, Sk, d, "bf16", causal, seed=31000 + Sq + Sk + Hq,
                                         want_lse=True))
    log(f"  {stats}")


# bf16 at d = 64, grids of at most 768 workgroups over at least 1024 keys: the
# eight-wave ping-pong kernel, each workgroup's key tiles in two halves run in
# anti-phase and merged at the end. Odd and even tile counts (17 tiles of 1030
# keys, 18 of 1100), ragged unmasked tails, a causal offset that is not a
# multiple of 32 (rows of one wave that do and do not see the second half's
# first tile), the second half hidden from whole waves (first q-tile; Sq < Sk
# with waves past Sq), GQA and MQA, and the 768-workgroup boundary.
PP64_FORMS = [
    (1, 4, 2, 1000, 1040, True), (1, 4, 4, 1030, 1030, True), (2, 4, 2, 300, 1100, False),
    (1, 8, 2, 130, 1500, True), (1, 8, 1, 1024, 1024, True), (2, 3, 1, 2000, 2000, False),
    (2, 48, 12, 1024, 1024, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal", PP64_FORMS)
def test_bf16_d64_ping_pong(gpu, B, Hq, Hkv, Sq, Sk, causal):
    stats = _run_full(sdpa_inputs.custom(B, Hq, Hkv, Sq, Sk, 64, "bf16", causal, seed=32000 + Sq + Sk + Hq,
                                         want_lse=True))
    log(f"  {stats}")


# The same kernel on e4m3 inputs (scores on the fp8 matrix cores, V widened
# exactly to bf16 on its way into LDS, P.V in bf16), which runs from 1024 keys
# on any grid: the forms above that cover odd tile counts, ragged tails, hidden
# second halves and GQA/MQA, and a grid of 1024 workgroups.
FP8_PP64_FORMS = [(1, 4, 2, 1000, 1040, True), (2, 4, 2, 300, 1100, False), (1, 8, 2, 130, 1500, True),
                  (1, 8, 1, 1024, 1024, True), (2, 3, 1, 2000, 2000, False), (8, 16, 4, 1024, 1024, False)]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal", FP8_PP64_FORMS)
def test_fp8_d64_ping_pong(gpu, B, Hq, Hkv, Sq, Sk, causal):
    stats = _run_full(sdpa_inputs.custom(B, Hq, Hkv, Sq, Sk, 64, "fp8", causal, seed=33000 + Sq + Sk + Hq,
                                         want_lse=True))
    log(f"  {stats}")


# bf16 at d = 128 on at most 256 q-tiles of 128 rows (512 causal): the same
# kernel, there chosen over the 256-row ping-pong kernel. One key (group 1 with
# no tile), a single ragged tile, odd and even tile counts, Sq < Sk under the
# causal mask with an offset that is not a multiple of 32, GQA, MQA and an odd
# group, and both sides of each boundary (unmasked 256: this kernel, 288: the
# other; causal 512 and 544).
PP128_FORMS = [
    (1, 4, 1, 1, 1, False), (1, 4, 4, 33, 33, True), (1, 4, 2, 200, 130, False), (1, 8, 2, 1000, 1000, True),
    (2, 8, 2, 700, 3000, True), (2, 3, 1, 130, 2000, False), (4, 8, 8, 1024, 1024, False),
    (4, 8, 8, 1025, 1025, False), (4, 8, 8, 2048, 2048, True), (4, 8, 8, 2049, 2049, True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal", PP128_FORMS)
def test_bf16_d128_key_halves(gpu, B, Hq, Hkv, Sq, Sk, causal):
    stats = _run_full(sdpa_inputs.custom(B, Hq, Hkv, Sq, Sk, 128, "bf16", causal, seed=34000 + Sq + Sk + Hq,
                                         want_lse=True))
    log(f"  {stats}")


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal", PP128_FORMS)
def test_fp8_d128_key_halves(gpu, B, Hq, Hkv, Sq, Sk, causal):
    """The same forms on e4m3 inputs: two fp8 score MFMAs per 32-key block, V
    widened to bf16 in 32 codes per lane (past each boundary the 256-row fp8 kernel)."""
    stats = _run_full(sdpa_inputs.custom(B, Hq, Hkv, Sq, Sk, 128, "fp8", causal, seed=35000 + Sq + Sk + Hq,
                                         want_lse=True))
    log(f"  {stats}")


# e4m3 at d = 32 and 64 below 1024 keys on grids of at most 256 workgroups of
# 128 rows with at least 384 keys: the four-wave fp8 kernel's eight-wave key
# split. Odd tile counts (3 tiles of 128: two in the first half), Sq < Sk with
# the second half hidden from the first rows under the causal mask, GQA, MQA
# and an odd group; the last form (288 workgroups) runs the four-wave form.
FP8_SPLIT_FORMS = [(2, 4, 4, 384, 384, True), (1, 4, 2, 1000, 1000, True), (2, 4, 2, 300, 700, False),
                   (1, 4, 2, 129, 900, True), (1, 8, 1, 500, 500, True), (2, 3, 1, 700, 700, False),
                   (4, 8, 8, 1000, 1000, False), (9, 8, 8, 500, 500, True)]


@pytest.mark.parametrize("d", (32, 64))
@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,causal", FP8_SPLIT_FORMS)
def test_fp8_key_split(gpu, d, B, Hq, Hkv, Sq, Sk, causal):
    stats = _run_full(sdpa_inputs.custom(B, Hq, Hkv, Sq, Sk, d, "fp8", causal, seed=36000 + Sq + Sk + Hq + d,
                                         want_lse=True))
    log(f"  {stats}")


def test_bf16_d128_key_halves_without_lse(gpu):
    """The d = 128 key-half kernel with no lse output requested."""
    _run_full(sdpa_inputs.custom(2, 4, 2, 700, 1300, 128, "bf16", True, seed=34500), want_lse=False)


def test_bf16_d64_ping_pong_without_lse(gpu):
    """The same kernel with no lse output requested (the store is skipped)."""
    _run_full(sdpa_inputs.custom(2, 4, 2, 700, 1300, 64, "bf16", True, seed=32500), want_lse=False)


@pytest.mark.parametrize("S,d,causal,heads", list(itertools.product([1, 17, 64, 65, 129, 257], (32, 64, 128),
                                                                    (False, True), [(4, 4), (4, 2), (4, 1)])))
def test_f32_tails(gpu, S, d, causal, heads):
    Hq, Hkv = heads
    _run_full(sdpa_inputs.custom(2, Hq, Hkv, S, S, d, "f32", causal, seed=2000 + S))


@pytest.mark.parametrize("B,H,S,d,causal", [(4, 8, 500, 64, False), (1, 8, 1000, 128, True), (4, 32, 512, 128, False),
                                            (4, 8, 1024, 64, True), (2, 24, 700, 64, True),
                                            (4, 8, 700, 64, False), (2, 24, 700, 64, False),
                                            (4, 16, 700, 128, False)])
def test_f32_grid_sizes(gpu, B, H, S, d, causal):
    """fp32 grids, in workgroups of 128 rows: 128 and 64 run the four-way key split with
    its LDS merge over many 128-key super-tiles (grids up to 128 split); 512 (d = 128)
    and 384 (d = 128, ragged tail) the four-wave kernel with the next tile prefetched
    into registers; 256 and 192 (d = 64, the latter unmasked with a ragged tail) the
    d = 64 prefetch variant; 288 (d = 64, causal and unmasked) the four-wave kernel
    without the prefetch. lse on."""
    _run_full(sdpa_inputs.custom(B, H, H, S, S, d, "f32", causal, seed=2500 + S + d, want_lse=True))


@pytest.mark.parametrize("S,d,causal,heads", list(itertools.product([1, 17, 63, 64, 65, 129, 257], (32, 64, 128),
                                                                    (False, True), HEADS)))
def test_fp8_tails(gpu, S, d, causal, heads):
    Hq, Hkv = heads
    _run_full(sdpa_inputs.custom(1, Hq, Hkv, S, S, d, "fp8", causal, seed=3000 + S))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("Sq,Sk", [(1, 300), (77, 5), (130, 257), (300, 64)])
def test_cross_attention_lengths(gpu, dtype, Sq, Sk):
    """Unmasked attention with Sq != Sk (query and key sequences of different length)."""
    _run_full(sdpa_inputs.custom(2, 4, 2, Sq, Sk, 128 if dtype != "f32" else 64, dtype, False, seed=Sq * 7 + Sk))


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("f32", 64), ("f32", 128), ("bf16", 32), ("bf16", 64),
                                     ("bf16", 128), ("fp8", 32), ("fp8", 64), ("fp8", 128)])
@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 300), (5, 64), (77, 200), (130, 257), (256, 1000), (300, 301)])
def test_causal_queries_are_the_last_positions(gpu, dtype, d, Sq, Sk):
    """Causal with Sq < Sk: query i sees keys j <= i + (Sk - Sq) (new queries against a longer key
    sequence); single-query decode shapes included. Element-wise against the oracle, lse on."""
    _run_full(sdpa_inputs.custom(2, 4, 2, Sq, Sk, d, dtype, True, seed=5000 + Sq * 3 + Sk, want_lse=True))


@pytest.mark.parametrize("d", [32, 64, 128])
def test_batch_and_heads_mapping(gpu, d):
    """Several batches and GQA groups at once, causal, lse on: groups of 4 and 2 query heads
    with the XCD-ordered work items (B * Hkv divisible by 8) and without."""
    for dtype in ("f32", "bf16", "fp8"):
        for B, Hq, Hkv, S in ((3, 12, 3, 200), (2, 16, 4, 333), (2, 16, 8, 333), (4, 12, 2, 129)):
            _run_full(sdpa_inputs.custom(B, Hq, Hkv, S, S, d, dtype, True, seed=55 + Hq + Hkv))


# ------------------------------------------------------------- golden fixtures

def test_golden_fixtures_fp32(gpu):
    """The hand-derived fixtures, zero-padded to d = 64 (padding leaves every dot product
    and the first output columns unchanged)."""
    import scaled_dot_product_18_amd as sdpa
    for c in load_all():
        log(f"[golden] {c['name']}")
        q, k, v = c["q"], c["k"], c["v"]
        d0 = q.shape[-1]

        def pad(x):
            y = np.zeros(x.shape[:-1] + (64,))
            y[..., :d0] = x
            return torch.from_numpy(y).to(torch.float32).cuda().contiguous()

        o, lse = sdpa.fwd(pad(q), pad(k), pad(v), causal=c["causal"], scale=c["scale"], want_lse=True)
        torch.cuda.synchronize()
        o = o.double().cpu().numpy()
        np.testing.assert_allclose(o[..., :d0], c["o"], atol=1e-5)
        np.testing.assert_array_equal(o[..., d0:], 0.0)
        np.testing.assert_allclose(lse.double().cpu().numpy(), c["lse"], atol=1e-5)


# ----------------------------------------------------------------- properties

@pytest.mark.parametrize("d", [32, 64, 128])
def test_large_score_offset(gpu, d):
    """Scores around 16 d (500 to 2000): the online softmax stays finite and matches the oracle."""
    import scaled_dot_product_18_amd as sdpa
    g = torch.Generator().manual_seed(5)
    S = 150
    base = torch.full((1, 2, S, d), 4.0)
    q = (base + 0.1 * torch.randn(1, 2, S, d, generator=g)).to(torch.bfloat16)
    k = (base + 0.1 * torch.randn(1, 2, S, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(1, 2, S, d, generator=g).to(torch.bfloat16)
    for causal in (False, True):
        o, lse = sdpa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=1.0, want_lse=True)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), 1.0, causal)
        assert np.all(l_ref > 12 * d)
        assert np.abs(o.double().cpu().numpy() - o_ref).max() <= TOL_O["bf16"]
        # fp32 scores of magnitude ~1e3 carry ~1e-5 relative rounding on top of the lse bound
        assert np.abs(lse.double().cpu().numpy() - l_ref).max() <= TOL_LSE["bf16"] + 1e-5 * np.abs(l_ref).max()


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_move_the_reference(gpu, d, causal):
    """Scores that grow along the key sequence by ~100 (natural-log units) force the
    running maximum to move many times mid-row; the result still matches the oracle."""
    import scaled_dot_product_18_amd as sdpa
    g = torch.Generator().manual_seed(77)
    S = 700
    q = torch.ones(1, 2, S, d) + 0.05 * torch.randn(1, 2, S, d, generator=g)
    ramp = torch.linspace(0.0, 1.0, S).view(1, 1, S, 1)
    k = 0.25 * torch.randn(1, 2, S, d, generator=g) + ramp * 100.0 / (d ** 0.5)
    v = torch.randn(1, 2, S, d, generator=g)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    scale = 1.0 / d ** 0.5
    o, lse = sdpa.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, want_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, causal)
    qd, kd = q.double(), k.double()
    rise = scale * ((qd[:, :, -1] * kd[:, :, -1]).sum(-1) - (qd[:, :, -1] * kd[:, :, 0]).sum(-1))
    assert float(rise.min()) > 50  # the last query's scores climb by > 50 along its keys
    assert np.abs(o.double().cpu().numpy() - o_ref).max() <= TOL_O["bf16"]
    assert np.abs(lse.double().cpu().numpy() - l_ref).max() <= TOL_LSE["bf16"] + 1e-5 * np.abs(l_ref).max()


def test_every_output_written(gpu):
    """Outputs pre-filled with NaN are overwritten everywhere (tails included)."""
    for dtype in ("f32", "bf16", "fp8"):
        w = sdpa_inputs.custom(2, 4, 2, 131, 131, 128, dtype, True, seed=9)
        dev = to_device(sdpa_inputs.make_inputs(w))
        out = torch.full((2, 4, 131, 128), float("nan"), dtype=torch.float32 if dtype == "f32" else torch.bfloat16,
                         device="cuda")
        lse = torch.full((2, 4, 131), float("nan"), device="cuda")
        run_gpu(w, dev, out=out, lse_out=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_deterministic(gpu):
    """Bitwise identical results across repeated calls (no atomics, fixed reduction order)."""
    w = sdpa_inputs.custom(2, 8, 2, 517, 517, 128, "bf16", True, seed=11)
    dev = to_device(sdpa_inputs.make_inputs(w))
    o1, l1 = run_gpu(w, dev)
    o2, l2 = run_gpu(w, dev)
    for _ in range(3):
        o3, l3 = run_gpu(w, dev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(o1, o3) and torch.equal(l1, l2) and torch.equal(l1, l3)


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("f32", 64), ("bf16", 32), ("bf16", 64), ("bf16", 128), ("fp8", 32),
                                     ("fp8", 64), ("fp8", 128)])
def test_gqa_equals_mha_on_repeated_kv(gpu, dtype, d):
    """GQA/MQA output is bit-identical to MHA on host-repeated K/V heads."""
    for Hkv in (2, 1):
        w = sdpa_inputs.custom(2, 8, Hkv, 190, 190, d, dtype, True, seed=21)
        inp = sdpa_inputs.make_inputs(w)
        o_g, l_g = run_gpu(w, to_device(inp))
        G = 8 // Hkv
        rep = dict(inp, k=inp["k"].repeat_interleave(G, dim=1).contiguous(),
                   v=inp["v"].repeat_interleave(G, dim=1).contiguous())
        w_m = sdpa_inputs.custom(2, 8, 8, 190, 190, d, dtype, True, seed=21)
        o_m, l_m = run_gpu(w_m, to_device(rep))
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_m) and torch.equal(l_g, l_m)


def test_causal_first_row_is_v0(gpu):
    """Causal row 0 attends only to key 0: O[...,0,:] = V[...,0,:] exactly, lse = scale q0.k0."""
    w = sdpa_inputs.custom(2, 4, 4, 300, 300, 128, "bf16", True, seed=31)
    inp = sdpa_inputs.make_inputs(w)
    o, lse = run_gpu(w, to_device(inp))
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0].cpu(), inp["v"][:, :, 0])
    s0 = (inp["q"][:, :, 0].double() * inp["k"][:, :, 0].double()).sum(-1) * w.scale
    assert torch.allclose(lse[:, :, 0].cpu().double(), s0, atol=1e-4)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_lse_optional(gpu, d):
    w = sdpa_inputs.custom(1, 4, 4, 100, 100, d, "bf16", False, seed=41)
    dev = to_device(sdpa_inputs.make_inputs(w))
    o1, lse = run_gpu(w, dev, want_lse=False)
    o2, _ = run_gpu(w, dev, want_lse=True)
    torch.cuda.synchronize()
    assert lse is None and torch.equal(o1, o2)


def test_errors_raise_through_python(gpu):
    import scaled_dot_product_18_amd as sdpa
    x = torch.zeros(1, 3, 8, 64, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdpa.AttnError, match="ATTN_ERR_HEADS"):
        sdpa.fwd(x, kv, kv)
    for bad_d in (16, 48, 96, 256):
        y = torch.zeros(1, 2, 8, bad_d, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(sdpa.AttnError, match="ATTN_ERR_HEADDIM"):
            sdpa.fwd(y, y, y)
    z = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    z9 = torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdpa.AttnError, match="ATTN_ERR_CAUSAL_SHAPE"):
        sdpa.fwd(z9, z, z, causal=True)


# ----------------------------------------------- full-size workloads, sampled rows

# Rows per head: the first rows (where causal softmax is sharpest and fp8 error
# concentrates), tile edges of the launched kernel, the last rows and random rows.
# The 16k fp8 workload checks rows 0-511 of every head plus 2048 random rows per head.
SAMPLED = {"causal_mha_bf16_b8_h16_s2048_d128": (64, 64), "causal_gqa_bf16_b4_hq32_hkv8_s4096_d128": (64, 64),
           "causal_mqa_bf16_b4_hq32_hkv1_s4096_d128": (64, 64), "causal_fp8_b1_h32_s16384_d128": (512, 2048)}


@pytest.mark.parametrize("name", list(SAMPLED))
def test_full_size_workload_sampled(gpu, name):
    w = sdpa_inputs.WORKLOADS[name]
    first, n_random = SAMPLED[name]
    log(f"[parity-full] {name}: rows 0..{first - 1}, tile edges and {n_random} random rows per head")
    inp = sdpa_inputs.make_inputs(w)
    dev = to_device(inp)
    o, lse = run_gpu(w, dev, want_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    stats = check_sampled(w, inp, o, lse, n_random=n_random, first=first)
    log(f"  {stats}")


@pytest.mark.parametrize("name", ["kv_heads_2_bf16_b2_t4096", "causal_bf16_b4_t2048", "seq_len_bf16_b4_t1024"])
def test_codelab_sweep_shapes_sampled(gpu, name):
    """The codelab's own d = 64 sweep shapes that run the ping-pong kernel (1024+ keys), at
    their full size, on sampled rows: the first rows, tile edges, the last rows and random rows."""
    import bench
    w = {x.name: x for _, x in bench.sweep_shapes()}[name]
    log(f"[parity-sweep] {w.name}")
    inp = sdpa_inputs.make_inputs(w)
    o, lse = run_gpu(w, to_device(inp), want_lse=True)
    torch.cuda.synchronize()
    stats = check_sampled(w, inp, o, lse, n_random=48, first=32)
    log(f"  {stats}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_sampled_causal_queries_against_longer_keys(gpu, dtype):
    """Causal, Sq < Sk at a size checked on sampled rows: query i sees keys j <= i + (Sk - Sq)."""
    w = sdpa_inputs.custom(1, 8, 2, 2000, 6000, 128, dtype, True, seed=6001, want_lse=True)
    log(f"[parity-sampled] {w.name}")
    inp = sdpa_inputs.make_inputs(w)
    o, lse = run_gpu(w, to_device(inp), want_lse=True)
    torch.cuda.synchronize()
    stats = check_sampled(w, inp, o, lse, n_random=64, first=16)
    log(f"  {stats}")

"""The C ABI library (CPU only): it loads, exports every symbol include/attn.h
declares, and rejects invalid arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "attn.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", text, flags=re.M)))


def _header_enums():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return {name: int(val) for name, val in re.findall(r"(ATTN_\w+)\s*=\s*(-?\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    from scaled_dot_product_18_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail(f"{_lib.LIB_PATH} not built: run __graft_entry__.build()")
    return _lib


def test_header_declares_the_boundary():
    assert _header_functions() == ["attn_bwd", "attn_bwd_fp8", "attn_bwd_fp8_workspace_size",
                                   "attn_bwd_workspace_size", "attn_fwd", "attn_fwd_fp8",
                                   "attn_fwd_splitkv", "attn_fwd_splitkv_noalloc", "attn_fwd_splitkv_plan",
                                   "attn_fwd_strided", "attn_strerror", "attn_version"]


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lib.LIB_PATH)
    for name in _header_functions():
        assert hasattr(raw, name), f"{name} missing from {lib.LIB_PATH}"


def test_python_constants_match_header(lib):
    enums = _header_enums()
    assert enums["ATTN_F32"] == lib.ATTN_F32 and enums["ATTN_BF16"] == lib.ATTN_BF16
    assert enums["ATTN_FP8_E4M3"] == lib.ATTN_FP8_E4M3
    for code, name in lib.STATUS.items():
        assert enums[name] == code


def test_strerror_covers_every_status(lib):
    for code in lib.STATUS:
        assert lib.strerror(code) and lib.strerror(code) != "unknown status"
    assert lib.strerror(12345) == "unknown status"
    assert lib.load().attn_version() >= 100


# Fake, aligned, never-dereferenced addresses: every case below is rejected
# by host-side validation before the library touches the HIP runtime.
P = 0x10000


def _call(lib, q=P, k=P, v=P, o=P, lse=None, B=1, Hq=2, Hkv=1, Sq=8, Sk=8, d=64, scale=0.125, causal=0,
          dtype=1):
    return lib.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kwargs,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(Sq=0), -2), (dict(Sk=-3), -2), (dict(d=0), -2),
    (dict(Sq=1 << 30), -2),
    (dict(Hq=3, Hkv=2), -3),
    (dict(d=96), -4), (dict(d=256), -4), (dict(d=16), -4), (dict(d=48), -4),
    (dict(causal=1, Sq=9, Sk=8), -5),
    (dict(dtype=3), -6), (dict(dtype=-1), -6),
    (dict(scale=0.0), -7), (dict(scale=-0.5), -7), (dict(scale=float("inf")), -7), (dict(scale=float("nan")), -7),
    (dict(q=P + 8), -8), (dict(o=P + 2), -8), (dict(lse=P + 4), -8),
])
def test_validation_errors(lib, kwargs, status):
    assert _call(lib, **kwargs) == status


def test_fp8_validation_errors(lib):
    f = lib.attn_fwd_fp8
    ok = dict(q8=P, k8=P, v8=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128, scale=0.1, causal=1,
              dq=1.0, dk=1.0, dv=1.0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q8"], a["k8"], a["v8"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"],
                 a["scale"], a["causal"], a["dq"], a["dk"], a["dv"], None)

    assert call(v8=None) == -1
    assert call(Hkv=3) == -3
    assert call(d=80) == -4
    assert call(Sq=9) == -5
    assert call(dq=0.0) == -7 and call(dk=float("nan")) == -7 and call(dv=-1.0) == -7
    assert call(scale=float("inf")) == -7
    assert call(k8=P + 1) == -8


def test_splitkv_validation_errors(lib):
    f = lib.load().attn_fwd_splitkv
    ok = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=1, Sq=1, Sk=4096, d=128, scale=0.1, causal=0,
              dtype=1, ns=8, ws=P, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"],
                 a["scale"], a["causal"], a["dtype"], a["ns"], a["ws"], a["ws_bytes"], None)

    assert call(dtype=0) == -6 and call(dtype=2) == -6
    assert call(o=None) == -1
    assert call(Sq=0) == -2
    assert call(Hkv=3) == -3
    assert call(d=96) == -4 and call(d=32) == -4
    assert call(causal=1, Sq=4097) == -5
    assert call(scale=0.0) == -7
    assert call(q=P + 4) == -8
    assert call(ns=-1) == -11 and call(ns=129) == -11
    assert call(ws=None) == -10
    assert call(ws=P + 8) == -10
    assert call(ws_bytes=1000) == -10
    st, n, nbytes = lib.attn_fwd_splitkv_plan(1, 4, 1, 1, 4096, 128, 8)
    assert (st, n) == (0, 8) and nbytes == 4 * 8 * 129 * 4
    assert call(ws_bytes=nbytes - 1) == -10


def test_splitkv_noalloc_validation_errors(lib):
    """The no-allocation variant checks its arguments like attn_fwd_splitkv, and rejects
    requests whose chunk partials exceed the static scratch (ATTN_SCRATCH_BYTES, 16 MiB)
    before any HIP call (so these run without a GPU)."""
    f = lib.load().attn_fwd_splitkv_noalloc
    ok = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=1, Sq=1, Sk=4096, d=128, scale=0.1, causal=0,
              dtype=1, ns=8)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"],
                 a["scale"], a["causal"], a["dtype"], a["ns"], None)

    assert call(dtype=0) == -6 and call(dtype=2) == -6
    assert call(o=None) == -1
    assert call(Sq=0) == -2
    assert call(Hkv=3) == -3
    assert call(d=96) == -4 and call(d=32) == -4
    assert call(causal=1, Sq=4097) == -5
    assert call(scale=0.0) == -7
    assert call(q=P + 4) == -8
    assert call(ns=-1) == -11 and call(ns=129) == -11
    # B*Hq*Sq*splits*(d+1)*4 bytes: 64*32*8*128*129*4 > 16 MiB; the plan agrees
    big = dict(B=64, Hq=32, Hkv=8, Sq=8, Sk=32768, ns=128)
    st, n, nbytes = lib.attn_fwd_splitkv_plan(64, 32, 8, 8, 32768, 128, 128)
    assert st == 0 and nbytes > 16 << 20
    assert call(**big) == -13
    assert "16 MiB" in lib.strerror(-13)


@pytest.mark.parametrize("sizes,ns", [((4, 32, 8, 1, 4096, 128), 0), ((4, 32, 32, 1, 4096, 128), 0),
                                      ((1, 32, 8, 16, 32768, 128), 0), ((32, 12, 12, 196, 196, 64), 0),
                                      ((1, 1, 1, 1, 1, 64), 0), ((2, 8, 2, 5, 1500, 128), 7),
                                      ((2, 8, 2, 5, 1500, 128), 128), ((1, 2, 1, 3, 100, 64), 128)])
def test_splitkv_plan(lib, sizes, ns):
    """Chunk counts: within [1, 128], within ceil(Sk / 32) (a chunk holds a multiple of 32
    keys), no empty chunk, at most what was asked for; the workspace holds fp32 partial
    outputs and log-sum-exps of every row and chunk, none for one chunk."""
    B, Hq, Hkv, Sq, Sk, d = sizes
    st, n, nbytes = lib.attn_fwd_splitkv_plan(B, Hq, Hkv, Sq, Sk, d, ns)
    assert st == 0
    assert 1 <= n <= min(128, -(-Sk // 32))
    if ns:
        assert n <= ns
    chunk = -(-(-(-Sk // max(n, 1))) // 32) * 32
    assert (n - 1) * chunk < Sk <= n * chunk or n == 1
    assert nbytes == (B * Hq * Sq * n * (d + 1) * 4 if n > 1 else 0)
    # The default fills the GPU: at least 256 workgroups or 256 keys per chunk.
    if ns == 0:
        items = B * Hkv * -(-(Hq // Hkv) * Sq // 32)
        assert items * n >= 256 or n == min(128, -(-Sk // 256)) or n == -(-Sk // 32)


def test_bwd_validation_errors(lib):
    f = lib.load().attn_bwd
    ok = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128, scale=0.1,
              causal=1, dtype=1, ws=P, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"], a["Hq"],
                 a["Hkv"], a["Sq"], a["Sk"], a["d"], a["scale"], a["causal"], a["dtype"], a["ws"], a["ws_bytes"],
                 None)

    assert call(dtype=2) == -6 and call(dtype=3) == -6
    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert call(**{name: None}) == -1, name
    assert call(Sk=0) == -2
    assert call(Hkv=3) == -3
    assert call(d=32) == -4 and call(d=48) == -4 and call(dtype=0, d=48) == -4  # bf16: 64, 128; fp32: 32, 64, 128
    assert call(Sq=9) == -5
    assert call(scale=float("nan")) == -7
    assert call(dk=P + 2) == -8 and call(do=P + 8) == -8
    assert call(ws=None) == -10 and call(ws=P + 4) == -10
    st, nbytes = lib.attn_bwd_workspace_size(1, 4, 2, 8, 8, 128)
    assert st == 0 and nbytes == 2 * 4 * 8 * 4
    assert call(ws_bytes=nbytes - 1) == -10
    # MQA with 8 query heads: the dK/dV kernel splits them into 2 subsets of 4, whose
    # fp32 partial dK and dV follow the 16-byte aligned row statistics.
    st, nbytes = lib.attn_bwd_workspace_size(1, 8, 1, 8, 8, 128)
    assert st == 0 and nbytes == 2 * 8 * 8 * 4 + 2 * 2 * 8 * 128 * 4
    st, nbytes = lib.attn_bwd_workspace_size(1, 4, 1, 8, 8, 128)  # 4 heads: no split
    assert st == 0 and nbytes == 2 * 4 * 8 * 4
    assert lib.attn_bwd_workspace_size(1, 3, 2, 8, 8, 128)[0] == -3
    assert lib.attn_bwd_workspace_size(1, 4, 2, 8, 8, 96)[0] == -4


def test_bwd_fp8_validation_errors(lib):
    f = lib.load().attn_bwd_fp8
    ok = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Sq=8, Sk=8, d=128, scale=0.1,
              causal=1, dsq=0.01, dsk=0.02, dsv=0.03, dsdo=1e-4, ws=P, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["B"], a["Hq"],
                 a["Hkv"], a["Sq"], a["Sk"], a["d"], a["scale"], a["causal"], a["dsq"], a["dsk"], a["dsv"],
                 a["dsdo"], a["ws"], a["ws_bytes"], None)

    for name in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert call(**{name: None}) == -1, name
    assert call(B=0) == -2
    assert call(Hkv=3) == -3
    assert call(d=32) == -4
    assert call(Sq=9) == -5
    for name in ("dsq", "dsk", "dsv", "dsdo"):
        assert call(**{name: 0.0}) == -7 and call(**{name: float("inf")}) == -7, name
    assert call(scale=-1.0) == -7
    assert call(dq=P + 2) == -8
    # workspace: the bf16 backward's, then bf16 copies of q8, dout8 (4*8*128 codes each)
    # and k8, v8 (2*8*128 codes each), every region from a 16-byte boundary
    st, nbytes = lib.attn_bwd_fp8_workspace_size(1, 4, 2, 8, 8, 128)
    assert st == 0 and nbytes == 2 * 4 * 8 * 4 + 2 * (2 * 4 * 8 * 128) + 2 * (2 * 2 * 8 * 128)
    assert call(ws=None) == -10 and call(ws=P + 8) == -10 and call(ws_bytes=nbytes - 1) == -10
    assert lib.attn_bwd_fp8_workspace_size(1, 4, 2, 8, 8, 32)[0] == -4


def test_strided_validation_errors(lib):
    """attn_fwd_strided rejects unusable strides (and the shared errors) before any HIP call."""
    B, Hq, Hkv, S, d = 2, 4, 2, 8, 64
    bshd_q = [S * Hq * d, d, Hq * d]
    bshd_kv = [S * Hkv * d, d, Hkv * d]
    good = bshd_q + bshd_kv + bshd_kv + bshd_q

    def call(strides=good, dtype=1, d=d, dq=1.0, **kw):
        a = dict(q=P, k=P, v=P, o=P, lse=None, causal=0, scale=0.125)
        a.update(kw)
        return lib.attn_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], B, Hq, Hkv, S, S, d, strides,
                                    a["scale"], a["causal"], dtype, dq, 1.0, 1.0, None)

    def with_(i, x):
        t = list(good)
        t[i] = x
        return t

    assert call(with_(2, d - 8)) == -12          # overlapping rows of q
    assert call(with_(5, -64)) == -12            # negative position stride of k
    assert call(with_(1, 4)) == -12              # head stride of 8 bytes: rows not 16-byte aligned
    assert call(with_(11, 1 << 30)) == -12       # a head of o spans more than 2 GiB
    assert call(with_(0, -1)) == -12
    assert call(dtype=0, dq=2.0) == -7           # descales other than 1 need fp8
    assert call(q=None) == -1 and call(d=96) == -4 and call(dtype=5) == -6
    assert call(causal=1, q=P + 4) == -8
    raw = lib.load().attn_fwd_strided
    assert raw(P, P, P, P, None, 1, 1, 1, 8, 8, 64, None, 0.1, 0, 1, 1.0, 1.0, 1.0, None) == -1


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    import scaled_dot_product_18_amd as sdpa
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        sdpa.fwd(x, x, x)
    with pytest.raises(ValueError):
        sdpa.fwd(x.to(torch.float16), x.to(torch.float16), x.to(torch.float16))
    with pytest.raises(ValueError):
        sdpa.fwd_fp8(x, x, x, 1.0, 1.0, 1.0)


def test_product_path_does_not_import_the_oracle():
    """The package never imports the oracle or the input generator."""
    pkg = os.path.join(ROOT, "scaled_dot_product_18_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+(oracle|sdpa_inputs)\b", text, flags=re.M), fn
                assert "oracle/" not in text, fn


def test_mfma_peak_library_is_built_apart_from_the_boundary():
    """The matrix-core microbenchmark (bench.py --mfma-peak) lives in its own library: it exports
    its launcher, and the attention library does not."""
    from scaled_dot_product_18_amd import _lib, build
    if not os.path.exists(build.PEAK_LIB_PATH):
        pytest.fail(f"{build.PEAK_LIB_PATH} not built: run __graft_entry__.build()")
    assert hasattr(ctypes.CDLL(build.PEAK_LIB_PATH), "mfma_peak_launch")
    assert not hasattr(ctypes.CDLL(_lib.LIB_PATH), "mfma_peak_launch")

"""bench.py's contract on the CPU: no multi-GPU run, the kernel it reports for
each workload is the one the library launches, and every workload has its
kernel-trace and HBM-counter summaries under profiles/."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import sdpa_inputs  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_names_follow_the_launch_dispatch():
    """The dominant kernel per workload, as the launchers pick it: the eight-wave
    ping-pong kernels at d=128 (the key-half one on small grids), the four-wave
    kernels at d=64, the fp32 key-split kernel for grids up to 128 workgroups of
    128 query rows."""
    W = sdpa_inputs.WORKLOADS
    assert bench.kernel_name(W["single_head_f32_s128_d64"]) == "attn_fwd_f32_split_kernel"
    assert bench.kernel_name(W["vit_b16_bf16_b32_h12_s196_d64"]) == "attn_fwd_bf16_kernel"
    assert bench.kernel_name(W["causal_gqa_bf16_b4_hq32_hkv8_s4096_d128"]) == "attn_fwd_bf16_pp_kernel"
    assert bench.kernel_name(W["causal_fp8_b1_h32_s16384_d128"]) == "attn_fwd_fp8_pp_kernel"
    assert bench.kernel_name(W["decode_gqa_bf16_b4_hq32_hkv8_sk32768_d128"]) == "attn_fwd_splitkv_kernel"
    assert bench.kernel_name(W["bwd_causal_gqa_bf16_b4_hq32_hkv8_s4096_d128"]) == "attn_bwd_dkdv_kernel"
    # the fp32 switch: 128 workgroups split the keys, 129 do not
    f32 = lambda B, H, S: sdpa_inputs.custom(B, H, H, S, S, 64, "f32", False, seed=0)  # noqa: E731
    assert bench.kernel_name(f32(1, 128, 128)) == "attn_fwd_f32_split_kernel"
    assert bench.kernel_name(f32(1, 129, 128)) == "attn_fwd_f32_kernel"
    assert bench.kernel_name(f32(1, 1, 32)) == "attn_fwd_f32_kernel"  # one key tile: nothing to split
    # d = 128 key halves: at most 256 q-tiles of 128 rows unmasked, 512 causal, whatever the KV heads
    w128 = lambda dt, Hkv, S, c: sdpa_inputs.custom(4, 8, Hkv, S, S, 128, dt, c, seed=0)  # noqa: E731
    for dt, big in (("bf16", "attn_fwd_bf16_pp_kernel"), ("fp8", "attn_fwd_fp8_pp_kernel")):
        for Hkv in (8, 2):
            assert bench.kernel_name(w128(dt, Hkv, 1024, False)) == "attn_fwd_ppk_kernel"
            assert bench.kernel_name(w128(dt, Hkv, 1025, False)) == big
            assert bench.kernel_name(w128(dt, Hkv, 2048, True)) == "attn_fwd_ppk_kernel"
            assert bench.kernel_name(w128(dt, Hkv, 2049, True)) == big


def test_every_kernel_name_has_a_source():
    for w in sdpa_inputs.WORKLOADS.values():
        src = bench.KERNEL_SOURCES[bench.kernel_name(w)]
        assert os.path.exists(os.path.join(bench.CSRC, src))
        src_text = open(os.path.join(bench.CSRC, src)).read()
        assert bench.kernel_name(w) in src_text


@pytest.mark.parametrize("name", sorted(sdpa_inputs.WORKLOADS))
def test_every_workload_has_profile_summaries(name):
    w = sdpa_inputs.WORKLOADS[name]
    kern = bench.kernel_name(w)
    for kind in ("trace", "hbm"):
        path = os.path.join(ROOT, "profiles", f"{kern}_{name}_{kind}.txt")
        assert os.path.exists(path), path
        text = open(path).read()
        assert "rocprofv3" in text and kern in text

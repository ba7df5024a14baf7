"""Fused scaled dot-product attention forward for AMD Instinct MI355X (gfx950).

    o, lse = fwd(q, k, v, causal=True, want_lse=True)

computes softmax(scale * Q K^T [+ causal mask]) V in one fused HIP kernel
(codelab "Accelerate attention on GPU with cuDNN and TransformerEngine",
intro and sections 4, 7, 9; article "Self-attention, CUDA kernels and
FlashAttention", section 3). Tensors are [B, H, S, d] on the GPU, or the
codelab's (B, T, N, H) with ``layout="bshd"``; any strides with contiguous
head dimension are read in place. K and V may have fewer heads than Q
(GQA/MQA, query head h reads KV head h // (Hq/Hkv)).

This module only marshals arguments into the C ABI of libsdpa18.so
(include/attn.h); PyTorch supplies device memory and the current stream.
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import AttnError, ATTN_BF16, ATTN_F32, ATTN_FP8_E4M3  # noqa: F401

__all__ = ["fwd", "fwd_fp8", "fwd_splitkv", "splitkv_plan", "bwd", "bwd_fp8", "AttnError", "library_path", "version",
           "require_library"]

_DTYPES = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}


def library_path() -> str:
    return _lib.LIB_PATH


def version() -> int:
    return _lib.load().attn_version()


def _shapes(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, S, d]")
    if k.shape != v.shape:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} differ")
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Sk, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"q {tuple(q.shape)} does not match k {tuple(k.shape)}")
    for t in (q, k, v):
        if not t.is_cuda:
            raise ValueError("inputs must be GPU tensors")
        if t.stride(-1) != 1:
            raise ValueError("the head dimension of every input must be contiguous (stride 1)")
        if t.device != q.device:
            raise ValueError("inputs must be on one device")
    return B, Hq, Hkv, Sq, Sk, d


def _dense_only(*ts) -> None:
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("this entry point takes contiguous [B, H, S, d] tensors")


def _as_bhsd(layout: str, *ts):
    """Views in the library's [B, H, S, d] order: "bshd" tensors (the codelab's (B, T, N, H)) are
    transposed as views, never copied."""
    if layout == "bhsd":
        return ts
    if layout == "bshd":
        return tuple(t.transpose(1, 2) for t in ts)
    raise ValueError(f"layout must be 'bhsd' or 'bshd', got {layout!r}")


def _outputs(q, B, Hq, Sq, d, out_dtype, want_lse, out, lse_out, layout="bhsd"):
    if out is None:
        if layout == "bshd":
            out = torch.empty((B, Sq, Hq, d), dtype=out_dtype, device=q.device).transpose(1, 2)
        else:
            out = torch.empty((B, Hq, Sq, d), dtype=out_dtype, device=q.device)
    elif out.shape != (B, Hq, Sq, d) or out.dtype != out_dtype or out.stride(-1) != 1 or out.device != q.device:
        raise ValueError("out has the wrong shape, dtype, layout or device")
    lse = None
    if want_lse or lse_out is not None:
        lse = lse_out if lse_out is not None else torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
        if lse.shape != (B, Hq, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse_out must be a contiguous float32 [B, Hq, Sq] tensor")
    return out, lse


def _strides(*ts):
    return [x for t in ts for x in (t.stride(0), t.stride(1), t.stride(2))]


def _launch(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, dtype, descales):
    """attn_fwd / attn_fwd_fp8 for dense tensors, attn_fwd_strided otherwise."""
    stream = torch.cuda.current_stream(q.device).cuda_stream
    lp = lse.data_ptr() if lse is not None else None
    if all(t.is_contiguous() for t in (q, k, v, out)):
        if dtype == ATTN_FP8_E4M3:
            return _lib.attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp, B, Hq, Hkv, Sq, Sk,
                                     d, scale, causal, *descales, stream)
        return _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp, B, Hq, Hkv, Sq, Sk, d,
                             scale, causal, dtype, stream)
    return _lib.attn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lp, B, Hq, Hkv, Sq, Sk, d,
                                 _strides(q, k, v, out), scale, causal, dtype, *descales, stream)


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False, scale: Optional[float] = None,
        want_lse: bool = False, out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
        layout: str = "bhsd") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused attention forward for float32 or bfloat16 inputs.

    scale defaults to 1/sqrt(d). ``layout="bhsd"`` takes [B, H, S, d] tensors;
    ``layout="bshd"`` takes the codelab's (B, T, N, H) and returns o in that
    layout. Strided views are read in place (the head dimension must be
    contiguous). Returns (o, lse) with o in the input dtype and lse float32
    [B, Hq, Sq] (natural log) or None. Enqueued on the current stream; nothing
    waits.
    """
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"fwd takes float32 or bfloat16 q/k/v of one dtype, got {q.dtype}/{k.dtype}/{v.dtype}")
    q, k, v = _as_bhsd(layout, q, k, v)
    if out is not None:
        (out,) = _as_bhsd(layout, out)
    B, Hq, Hkv, Sq, Sk, d = _shapes(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, B, Hq, Sq, d, q.dtype, want_lse, out, lse_out, layout)
    _lib.check(_launch(q, k, v, out, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, _DTYPES[q.dtype], (1.0, 1.0, 1.0)))
    (out,) = _as_bhsd(layout, out)
    return out, lse


def fwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, descale_q: float, descale_k: float,
            descale_v: float, *, causal: bool = False, scale: Optional[float] = None, want_lse: bool = False,
            out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
            layout: str = "bhsd") -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused attention forward on fp8-e4m3fn codes (uint8 or float8_e4m3fn tensors)
    with per-tensor descales; bfloat16 output. Other arguments as :func:`fwd`."""
    ok = (torch.uint8, torch.float8_e4m3fn)
    if q8.dtype not in ok or k8.dtype not in ok or v8.dtype not in ok:
        raise ValueError("fwd_fp8 takes uint8 or float8_e4m3fn codes")
    q8, k8, v8 = _as_bhsd(layout, q8, k8, v8)
    if out is not None:
        (out,) = _as_bhsd(layout, out)
    B, Hq, Hkv, Sq, Sk, d = _shapes(q8, k8, v8)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q8, B, Hq, Sq, d, torch.bfloat16, want_lse, out, lse_out, layout)
    _lib.check(_launch(q8, k8, v8, out, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, ATTN_FP8_E4M3,
                       (float(descale_q), float(descale_k), float(descale_v))))
    (out,) = _as_bhsd(layout, out)
    return out, lse


def splitkv_plan(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int, num_splits: int = 0) -> Tuple[int, int]:
    """(key chunks, workspace bytes) that :func:`fwd_splitkv` uses for these sizes."""
    st, n, nbytes = _lib.attn_fwd_splitkv_plan(B, Hq, Hkv, Sq, Sk, d, num_splits)
    _lib.check(st)
    return n, nbytes


def fwd_splitkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                scale: Optional[float] = None, want_lse: bool = False, num_splits: int = 0,
                out: Optional[torch.Tensor] = None, lse_out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Split-KV attention forward for bfloat16 inputs: the same result as :func:`fwd`,
    computed for few queries against many keys (decoding against a KV cache).

    The keys are cut into ``num_splits`` chunks (0 = the library's choice) that
    run in parallel and merge exactly through their log-sum-exps. ``workspace``
    (a device tensor of at least ``splitkv_plan(...)[1]`` bytes) is allocated
    here when not given. Other arguments as :func:`fwd`.
    """
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"fwd_splitkv takes bfloat16 q/k/v, got {q.dtype}/{k.dtype}/{v.dtype}")
    B, Hq, Hkv, Sq, Sk, d = _shapes(q, k, v)
    _dense_only(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out, lse = _outputs(q, B, Hq, Sq, d, q.dtype, want_lse, out, lse_out)
    _dense_only(out)
    _, nbytes = splitkv_plan(B, Hq, Hkv, Sq, Sk, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device) if nbytes else None
    elif not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _lib.check(_lib.attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr() if lse is not None else None,
                                     B, Hq, Hkv, Sq, Sk, d, scale, causal, ATTN_BF16, int(num_splits),
                                     ws_ptr, ws_bytes, stream))
    return out, lse


def _check_bwd_shapes(q, o, dout, lse, B, Hq, Sq):
    for name, t in (("o", o), ("dout", dout)):
        if t.shape != q.shape or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous tensor of q's shape on q's device")
    if lse.shape != (B, Hq, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be the contiguous float32 [B, Hq, Sq] tensor the forward returned")


def _workspace(workspace, nbytes, device):
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if not workspace.is_cuda or workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
        dout: torch.Tensor, *, causal: bool = False, scale: Optional[float] = None,
        workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dq, dk, dv) of the attention forward for bfloat16 or float32 tensors.

    ``o`` and ``lse`` are what :func:`fwd` returned for (q, k, v) with
    ``want_lse=True`` and the same ``causal`` and ``scale``; ``dout`` is the
    gradient of the loss with respect to ``o``. dk and dv have k's shape (with
    GQA/MQA they sum over the query heads that share a KV head). ``workspace``
    is allocated here when not given.
    """
    dt = q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise ValueError(f"bwd takes bfloat16 or float32 tensors, q is {dt}")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != dt:
            raise ValueError(f"bwd takes tensors of one dtype: q is {dt}, {name} is {t.dtype}")
    B, Hq, Hkv, Sq, Sk, d = _shapes(q, k, v)
    _dense_only(q, k, v)
    _check_bwd_shapes(q, o, dout, lse, B, Hq, Sq)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st, nbytes = _lib.attn_bwd_workspace_size(B, Hq, Hkv, Sq, Sk, d)
    _lib.check(st)
    workspace = _workspace(workspace, nbytes, q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _lib.check(_lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                             lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                             B, Hq, Hkv, Sq, Sk, d, scale, causal, ATTN_BF16 if dt == torch.bfloat16 else ATTN_F32,
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream))
    return dq, dk, dv


def bwd_fp8(q8: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
            dout8: torch.Tensor, descale_q: float, descale_k: float, descale_v: float, descale_do: float, *,
            causal: bool = False, scale: Optional[float] = None,
            workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dq, dk, dv; bfloat16, real values) for fp8 inputs: e4m3fn codes
    q8/k8/v8 and e5m2 codes dout8 (uint8 tensors) with per-tensor descales, the
    bfloat16 ``o`` and float32 ``lse`` that :func:`fwd_fp8` returned."""
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8), ("dout8", dout8)):
        if t.dtype != torch.uint8:
            raise ValueError(f"bwd_fp8 takes uint8 fp8 codes, {name} is {t.dtype}")
    if o.dtype != torch.bfloat16:
        raise ValueError(f"bwd_fp8 takes the bfloat16 forward output, o is {o.dtype}")
    B, Hq, Hkv, Sq, Sk, d = _shapes(q8, k8, v8)
    _dense_only(q8, k8, v8)
    if dout8.shape != q8.shape or not dout8.is_contiguous() or dout8.device != q8.device:
        raise ValueError("dout8 must be a contiguous tensor of q8's shape on q8's device")
    if o.shape != q8.shape or not o.is_contiguous() or o.device != q8.device:
        raise ValueError("o must be a contiguous tensor of q8's shape on q8's device")
    if lse.shape != (B, Hq, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q8.device:
        raise ValueError("lse must be the contiguous float32 [B, Hq, Sq] tensor fwd_fp8 returned")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st, nbytes = _lib.attn_bwd_fp8_workspace_size(B, Hq, Hkv, Sq, Sk, d)
    _lib.check(st)
    workspace = _workspace(workspace, nbytes, q8.device)
    dq = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device)
    dk = torch.empty(k8.shape, dtype=torch.bfloat16, device=q8.device)
    dv = torch.empty(v8.shape, dtype=torch.bfloat16, device=q8.device)
    stream = torch.cuda.current_stream(q8.device).cuda_stream
    _lib.check(_lib.attn_bwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), dout8.data_ptr(),
                                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                 B, Hq, Hkv, Sq, Sk, d, scale, causal, float(descale_q), float(descale_k),
                                 float(descale_v), float(descale_do),
                                 workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream))
    return dq, dk, dv


def require_library() -> None:
    """Load libsdpa18.so now; raises RuntimeError if it is missing (there is no other path)."""
    _lib.load()

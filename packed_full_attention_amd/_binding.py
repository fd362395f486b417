"""ctypes binding of libh3attn (argument marshalling only).

Every step of the path runs in the HIP kernels behind the C ABI; this module
checks torch tensors (dtype, device, contiguity, shape), passes their device
pointers and torch's current stream, and turns a non-zero status into an
exception.  There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libh3attn.so")
HEAD_DIM = 128
H3A_OK, H3A_EINVAL, H3A_EUNSUPPORTED, H3A_EHIP = 0, 1, 2, 3
EXPORTED_SYMBOLS = ("h3attn_qk_prologue", "h3attn_forward", "h3attn_qk_prologue_scaled", "h3attn_vt_bytes",
                    "h3attn_v_transpose", "h3attn_forward_log2", "h3attn_forward_lse",
                    "h3attn_attention_backward_workspace_bytes", "h3attn_attention_backward",
                    "h3attn_qk_prologue_backward_workspace_bytes", "h3attn_qk_prologue_backward",
                    "h3attn_rope_table_bytes", "h3attn_k_prologue_table", "h3attn_forward_log2_qprologue",
                    "h3attn_forward_log2_lse", "h3attn_qk_prologue_backward_scaled",
                    "h3attn_attention_backward_noalloc", "h3attn_kv_prologue", "h3attn_kv_prologue_fp8",
                    "h3attn_forward_fp8_qprologue",
                    "h3attn_strerror", "h3attn_last_error", "h3attn_abi_version")

_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None


class H3AttnError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: status {status}: {message}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libh3attn.so and declare its signatures (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is not None and path == LIB_PATH:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m packed_full_attention_amd.build` (there is no fallback path)")
        lib = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        lib.h3attn_qk_prologue.argtypes = [vp, vp, vp, vp, vp, i64, i32, vp]
        lib.h3attn_qk_prologue.restype = ctypes.c_int
        lib.h3attn_forward.argtypes = [vp, vp, vp, vp, i64, i32, ctypes.c_float, vp]
        lib.h3attn_forward.restype = ctypes.c_int
        lib.h3attn_qk_prologue_scaled.argtypes = [vp, vp, vp, vp, vp, i64, i32, ctypes.c_float, vp]
        lib.h3attn_qk_prologue_scaled.restype = ctypes.c_int
        lib.h3attn_forward_log2.argtypes = [vp, vp, vp, vp, i64, i32, vp]
        lib.h3attn_forward_log2.restype = ctypes.c_int
        lib.h3attn_vt_bytes.argtypes = [i64, i32]
        lib.h3attn_vt_bytes.restype = i64
        lib.h3attn_v_transpose.argtypes = [vp, vp, i64, i32, vp]
        lib.h3attn_v_transpose.restype = ctypes.c_int
        lib.h3attn_forward_lse.argtypes = [vp, vp, vp, vp, vp, i64, i32, ctypes.c_float, vp]
        lib.h3attn_forward_lse.restype = ctypes.c_int
        lib.h3attn_attention_backward_workspace_bytes.argtypes = [i64, i32]
        lib.h3attn_attention_backward_workspace_bytes.restype = i64
        lib.h3attn_attention_backward.argtypes = [vp] * 10 + [i64, i32, ctypes.c_float, vp]
        lib.h3attn_attention_backward.restype = ctypes.c_int
        lib.h3attn_qk_prologue_backward_workspace_bytes.argtypes = [i64, i32]
        lib.h3attn_qk_prologue_backward_workspace_bytes.restype = i64
        lib.h3attn_qk_prologue_backward.argtypes = [vp] * 10 + [i64, i32, vp]
        lib.h3attn_qk_prologue_backward.restype = ctypes.c_int
        lib.h3attn_rope_table_bytes.argtypes = [i64, i32]
        lib.h3attn_rope_table_bytes.restype = i64
        lib.h3attn_k_prologue_table.argtypes = [vp, vp, vp, vp, i64, i32, vp]
        lib.h3attn_k_prologue_table.restype = ctypes.c_int
        lib.h3attn_forward_log2_qprologue.argtypes = [vp] * 6 + [i64, i32, ctypes.c_float, vp]
        lib.h3attn_forward_log2_qprologue.restype = ctypes.c_int
        lib.h3attn_forward_log2_lse.argtypes = [vp, vp, vp, vp, vp, i64, i32, vp]
        lib.h3attn_forward_log2_lse.restype = ctypes.c_int
        lib.h3attn_qk_prologue_backward_scaled.argtypes = [vp] * 10 + [i64, i32, ctypes.c_float, vp]
        lib.h3attn_qk_prologue_backward_scaled.restype = ctypes.c_int
        lib.h3attn_attention_backward_noalloc.argtypes = [vp] * 9 + [i64, i32, ctypes.c_float, vp]
        lib.h3attn_attention_backward_noalloc.restype = ctypes.c_int
        lib.h3attn_kv_prologue.argtypes = [vp] * 6 + [i64, i32, vp]
        lib.h3attn_kv_prologue.restype = ctypes.c_int
        lib.h3attn_kv_prologue_fp8.argtypes = [vp] * 7 + [i64, i32, vp]
        lib.h3attn_kv_prologue_fp8.restype = ctypes.c_int
        lib.h3attn_forward_fp8_qprologue.argtypes = [vp] * 6 + [i64, i32, ctypes.c_float, vp]
        lib.h3attn_forward_fp8_qprologue.restype = ctypes.c_int
        lib.h3attn_strerror.argtypes = [ctypes.c_int]
        lib.h3attn_strerror.restype = ctypes.c_char_p
        lib.h3attn_last_error.argtypes = []
        lib.h3attn_last_error.restype = ctypes.c_char_p
        lib.h3attn_abi_version.argtypes = []
        lib.h3attn_abi_version.restype = ctypes.c_int
        if path == LIB_PATH:
            _lib = lib
        return lib


def _raise_on(lib, fn: str, status: int) -> None:
    if status != H3A_OK:
        detail = lib.h3attn_last_error().decode()
        raise H3AttnError(fn, status, f"{lib.h3attn_strerror(status).decode()} ({detail})")


def _check_tensor(name, t, dtype, shape, device=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _lh(q):
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError(f"q must be a [L, H, {HEAD_DIM}] tensor")
    return int(q.shape[0]), int(q.shape[1])


def _prologue(fn: str, q, k, gamma_q, gamma_k, pos_thw, q_scale) -> None:
    import torch
    L, H = _lh(q)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, (L, H, HEAD_DIM))
    _check_tensor("k", k, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("gamma_q", gamma_q, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("gamma_k", gamma_k, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("pos_thw", pos_thw, torch.int32, (L, 3), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        args = (q.data_ptr(), k.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(), pos_thw.data_ptr(), L, H)
        if q_scale is None:
            st = lib.h3attn_qk_prologue(*args, stream)
        else:
            st = lib.h3attn_qk_prologue_scaled(*args, float(q_scale), stream)
    _raise_on(lib, fn, st)


def h3attn_qk_prologue(q, k, gamma_q, gamma_k, pos_thw) -> None:
    """In-place Q/K RMSNorm + MM-RoPE on bf16 [L, H, 128] q and k (see include/h3attn.h)."""
    _prologue("h3attn_qk_prologue", q, k, gamma_q, gamma_k, pos_thw, None)


def h3attn_qk_prologue_scaled(q, k, gamma_q, gamma_k, pos_thw, q_scale: float) -> None:
    """h3attn_qk_prologue with Q's output multiplied by q_scale before its bf16 rounding."""
    _prologue("h3attn_qk_prologue_scaled", q, k, gamma_q, gamma_k, pos_thw, q_scale)


def _forward(fn: str, q, k, v, out, scale):
    import torch
    L, H = _lh(q)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, (L, H, HEAD_DIM))
    _check_tensor("k", k, torch.bfloat16, (L, H, HEAD_DIM), dev)
    if scale is None:
        _check_tensor("vt", v, torch.bfloat16, (H, HEAD_DIM, padded_length(L)), dev)
    else:
        _check_tensor("v", v, torch.bfloat16, (L, H, HEAD_DIM), dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, torch.bfloat16, (L, H, HEAD_DIM), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), L, H)
        if scale is None:
            st = lib.h3attn_forward_log2(*args, stream)
        else:
            st = lib.h3attn_forward(*args, float(scale), stream)
    _raise_on(lib, fn, st)
    return out


def h3attn_forward(q, k, v, out=None, scale: Optional[float] = None):
    """Full bidirectional attention on bf16 [L, H, 128]; returns out (see include/h3attn.h)."""
    return _forward("h3attn_forward", q, k, v, out, 1.0 / math.sqrt(HEAD_DIM) if scale is None else scale)


def padded_length(L: int) -> int:
    """Lp: L rounded up to a multiple of 64 (the key dimension of vt)."""
    return (int(L) + 63) // 64 * 64


def h3attn_v_transpose(v, vt=None):
    """vt[h, c, j] = v[j, h, c] for j < L, zero for L <= j < Lp; returns vt (bf16 [H, 128, Lp])."""
    import torch
    L, H = _lh(v)
    dev = v.device
    _check_tensor("v", v, torch.bfloat16, (L, H, HEAD_DIM))
    if vt is None:
        vt = torch.empty(H, HEAD_DIM, padded_length(L), dtype=torch.bfloat16, device=dev)
    _check_tensor("vt", vt, torch.bfloat16, (H, HEAD_DIM, padded_length(L)), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.h3attn_v_transpose(v.data_ptr(), vt.data_ptr(), L, H, torch.cuda.current_stream(dev).cuda_stream)
    _raise_on(lib, "h3attn_v_transpose", st)
    return vt


def h3attn_forward_log2(q, k, vt, out=None):
    """Base-2 softmax attention (q carries the softmax scale times log2(e); V as vt from
    h3attn_v_transpose); returns out."""
    return _forward("h3attn_forward_log2", q, k, vt, out, None)


def h3attn_k_prologue_table(k, gamma_k, pos_thw, rope_cs=None):
    """In-place prologue of k alone (the bits h3attn_qk_prologue gives it) plus the
    per-token rotation table rope_cs, fp32 [L, 96] (cosines, then sines); returns rope_cs."""
    import torch
    L, H = _lh(k)
    dev = k.device
    _check_tensor("k", k, torch.bfloat16, (L, H, HEAD_DIM))
    _check_tensor("gamma_k", gamma_k, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("pos_thw", pos_thw, torch.int32, (L, 3), dev)
    if rope_cs is None:
        rope_cs = torch.empty(L, 96, dtype=torch.float32, device=dev)
    _check_tensor("rope_cs", rope_cs, torch.float32, (L, 96), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.h3attn_k_prologue_table(k.data_ptr(), gamma_k.data_ptr(), pos_thw.data_ptr(), rope_cs.data_ptr(),
                                         L, H, torch.cuda.current_stream(dev).cuda_stream)
    _raise_on(lib, "h3attn_k_prologue_table", st)
    return rope_cs


def h3attn_kv_prologue(k, v, gamma_k, pos_thw, rope_cs=None, vt=None):
    """h3attn_k_prologue_table and h3attn_v_transpose in one launch: k rewritten in place,
    returns (rope_cs fp32 [L, 96], vt bf16 [H, 128, Lp])."""
    import torch
    L, H = _lh(k)
    dev = k.device
    _check_tensor("k", k, torch.bfloat16, (L, H, HEAD_DIM))
    _check_tensor("v", v, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("gamma_k", gamma_k, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("pos_thw", pos_thw, torch.int32, (L, 3), dev)
    if rope_cs is None:
        rope_cs = torch.empty(L, 96, dtype=torch.float32, device=dev)
    if vt is None:
        vt = torch.empty(H, HEAD_DIM, padded_length(L), dtype=torch.bfloat16, device=dev)
    _check_tensor("rope_cs", rope_cs, torch.float32, (L, 96), dev)
    _check_tensor("vt", vt, torch.bfloat16, (H, HEAD_DIM, padded_length(L)), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.h3attn_kv_prologue(k.data_ptr(), v.data_ptr(), gamma_k.data_ptr(), pos_thw.data_ptr(),
                                    rope_cs.data_ptr(), vt.data_ptr(), L, H, torch.cuda.current_stream(dev).cuda_stream)
    _raise_on(lib, "h3attn_kv_prologue", st)
    return rope_cs, vt


def h3attn_kv_prologue_fp8(k, v, gamma_k, pos_thw, rope_cs=None, k8=None, vt=None):
    """The quantized-score path's prologue: returns (rope_cs fp32 [L, 96], k8 uint8 [L, H, 128]
    (K's prologue output / 4 as e4m3, channels in the kernel's order), vt bf16 [H, 128, Lp]);
    k is read only."""
    import torch
    L, H = _lh(k)
    dev = k.device
    _check_tensor("k", k, torch.bfloat16, (L, H, HEAD_DIM))
    _check_tensor("v", v, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("gamma_k", gamma_k, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("pos_thw", pos_thw, torch.int32, (L, 3), dev)
    if rope_cs is None:
        rope_cs = torch.empty(L, 96, dtype=torch.float32, device=dev)
    if k8 is None:
        k8 = torch.empty(L, H, HEAD_DIM, dtype=torch.uint8, device=dev)
    if vt is None:
        vt = torch.empty(H, HEAD_DIM, padded_length(L), dtype=torch.bfloat16, device=dev)
    _check_tensor("rope_cs", rope_cs, torch.float32, (L, 96), dev)
    _check_tensor("k8", k8, torch.uint8, (L, H, HEAD_DIM), dev)
    _check_tensor("vt", vt, torch.bfloat16, (H, HEAD_DIM, padded_length(L)), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.h3attn_kv_prologue_fp8(k.data_ptr(), v.data_ptr(), gamma_k.data_ptr(), pos_thw.data_ptr(),
                                        rope_cs.data_ptr(), k8.data_ptr(), vt.data_ptr(), L, H,
                                        torch.cuda.current_stream(dev).cuda_stream)
    _raise_on(lib, "h3attn_kv_prologue_fp8", st)
    return rope_cs, k8, vt


def h3attn_forward_fp8_qprologue(q, k8, vt, gamma_q, rope_cs, q_scale: float, out=None):
    """Quantized-score attention (e4m3 Q'K^T, see include/h3attn.h) of the raw q against
    h3attn_kv_prologue_fp8's k8 and vt; returns out."""
    import torch
    L, H = _lh(q)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, (L, H, HEAD_DIM))
    _check_tensor("k8", k8, torch.uint8, (L, H, HEAD_DIM), dev)
    _check_tensor("vt", vt, torch.bfloat16, (H, HEAD_DIM, padded_length(L)), dev)
    _check_tensor("gamma_q", gamma_q, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("rope_cs", rope_cs, torch.float32, (L, 96), dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, torch.bfloat16, (L, H, HEAD_DIM), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.h3attn_forward_fp8_qprologue(q.data_ptr(), k8.data_ptr(), vt.data_ptr(), out.data_ptr(),
                                              gamma_q.data_ptr(), rope_cs.data_ptr(), L, H, float(q_scale),
                                              torch.cuda.current_stream(dev).cuda_stream)
    _raise_on(lib, "h3attn_forward_fp8_qprologue", st)
    return out


def h3attn_forward_log2_qprologue(q, k, vt, gamma_q, rope_cs, q_scale: float, out=None):
    """h3attn_forward_log2 with Q's prologue (gamma_q, rope_cs, q_scale) applied inside
    the attention kernel to the raw q, which is not modified; returns out."""
    import torch
    L, H = _lh(q)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, (L, H, HEAD_DIM))
    _check_tensor("k", k, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("vt", vt, torch.bfloat16, (H, HEAD_DIM, padded_length(L)), dev)
    _check_tensor("gamma_q", gamma_q, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("rope_cs", rope_cs, torch.float32, (L, 96), dev)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor("out", out, torch.bfloat16, (L, H, HEAD_DIM), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.h3attn_forward_log2_qprologue(q.data_ptr(), k.data_ptr(), vt.data_ptr(), out.data_ptr(),
                                               gamma_q.data_ptr(), rope_cs.data_ptr(), L, H, float(q_scale),
                                               torch.cuda.current_stream(dev).cuda_stream)
    _raise_on(lib, "h3attn_forward_log2_qprologue", st)
    return out


def _forward_lse(fn, q, k, v, out, lse, scale):
    import torch
    L, H = _lh(q)
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("k", k, torch.bfloat16, (L, H, HEAD_DIM), dev)
    if scale is None:
        _check_tensor("vt", v, torch.bfloat16, (H, HEAD_DIM, padded_length(L)), dev)
    else:
        _check_tensor("v", v, torch.bfloat16, (L, H, HEAD_DIM), dev)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(H, L, dtype=torch.float32, device=dev) if lse is None else lse
    _check_tensor("out", out, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("lse", lse, torch.float32, (H, L), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), L, H)
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.h3attn_forward_log2_lse(*args, stream) if scale is None else lib.h3attn_forward_lse(*args, scale, stream)
    _raise_on(lib, fn, st)
    return out, lse


def h3attn_forward_lse(q, k, v, out=None, lse=None, scale: Optional[float] = None):
    """h3attn_forward that also returns each row's natural log-sum-exp, fp32 [H, L]:
    returns (out, lse)."""
    return _forward_lse("h3attn_forward_lse", q, k, v, out, lse,
                        1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale))


def h3attn_forward_log2_lse(q, k, vt, out=None, lse=None):
    """h3attn_forward_log2 that also returns each row's natural log-sum-exp, fp32 [H, L]:
    returns (out, lse)."""
    return _forward_lse("h3attn_forward_log2_lse", q, k, vt, out, lse, None)


def h3attn_attention_backward(q, k, v, out, dout, lse, dq=None, dk=None, dv=None, workspace=None,
                              scale: Optional[float] = None):
    """Gradients (dq, dk, dv), bf16 [L, H, 128], of h3attn_forward_lse's output given dout."""
    import torch
    L, H = _lh(q)
    dev = q.device
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_tensor(name, t, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("lse", lse, torch.float32, (H, L), dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, torch.bfloat16, (L, H, HEAD_DIM), dev)
    lib = load_library()
    nbytes = int(lib.h3attn_attention_backward_workspace_bytes(L, H))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.numel() * workspace.element_size() < nbytes or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous buffer of >= {nbytes} bytes on {dev}")
    with torch.cuda.device(dev):
        st = lib.h3attn_attention_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                           lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                           workspace.data_ptr(), L, H, scale,
                                           torch.cuda.current_stream(dev).cuda_stream)
    _raise_on(lib, "h3attn_attention_backward", st)
    return dq, dk, dv


def h3attn_attention_backward_noalloc(q, k, v, out, dout, lse, dq, dk, dv, scale: Optional[float] = None):
    """h3attn_attention_backward with the statistics in the library's own device
    array (no workspace, nothing allocated: dq, dk, dv must be given); writes
    dq, dk, dv and returns them."""
    import torch
    L, H = _lh(q)
    dev = q.device
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("lse", lse, torch.float32, (H, L), dev)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.h3attn_attention_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                   dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                                   dv.data_ptr(), L, H, scale,
                                                   torch.cuda.current_stream(dev).cuda_stream)
    _raise_on(lib, "h3attn_attention_backward_noalloc", st)
    return dq, dk, dv


def _prologue_backward(fn, q, k, gamma_q, gamma_k, pos_thw, dq, dk, dgamma_q, dgamma_k, workspace, q_scale):
    import torch
    L, H = _lh(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("dq", dq), ("dk", dk)):
        _check_tensor(name, t, torch.bfloat16, (L, H, HEAD_DIM), dev)
    _check_tensor("gamma_q", gamma_q, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("gamma_k", gamma_k, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("pos_thw", pos_thw, torch.int32, (L, 3), dev)
    dgamma_q = torch.empty(HEAD_DIM, dtype=torch.float32, device=dev) if dgamma_q is None else dgamma_q
    dgamma_k = torch.empty(HEAD_DIM, dtype=torch.float32, device=dev) if dgamma_k is None else dgamma_k
    _check_tensor("dgamma_q", dgamma_q, torch.float32, (HEAD_DIM,), dev)
    _check_tensor("dgamma_k", dgamma_k, torch.float32, (HEAD_DIM,), dev)
    lib = load_library()
    nbytes = int(lib.h3attn_qk_prologue_backward_workspace_bytes(L, H))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=dev)
    if workspace.device != dev or workspace.numel() * workspace.element_size() < nbytes or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous buffer of >= {nbytes} bytes on {dev}")
    with torch.cuda.device(dev):
        args = (q.data_ptr(), k.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(), pos_thw.data_ptr(), dq.data_ptr(),
                dk.data_ptr(), dgamma_q.data_ptr(), dgamma_k.data_ptr(), workspace.data_ptr(), L, H)
        stream = torch.cuda.current_stream(dev).cuda_stream
        if q_scale is None:
            st = lib.h3attn_qk_prologue_backward(*args, stream)
        else:
            st = lib.h3attn_qk_prologue_backward_scaled(*args, float(q_scale), stream)
    _raise_on(lib, fn, st)
    return dgamma_q, dgamma_k


def h3attn_qk_prologue_backward(q, k, gamma_q, gamma_k, pos_thw, dq, dk, dgamma_q=None, dgamma_k=None,
                                workspace=None):
    """In place: dq, dk (gradients w.r.t. the prologue outputs) become the gradients w.r.t. the
    raw q, k; returns (dgamma_q, dgamma_k), fp32 [128]."""
    return _prologue_backward("h3attn_qk_prologue_backward", q, k, gamma_q, gamma_k, pos_thw, dq, dk, dgamma_q,
                              dgamma_k, workspace, None)


def h3attn_qk_prologue_backward_scaled(q, k, gamma_q, gamma_k, pos_thw, dq, dk, q_scale: float, dgamma_q=None,
                                       dgamma_k=None, workspace=None):
    """h3attn_qk_prologue_backward of h3attn_qk_prologue_scaled's prologue (dq: the gradient
    w.r.t. Q's scaled output); returns (dgamma_q, dgamma_k)."""
    return _prologue_backward("h3attn_qk_prologue_backward_scaled", q, k, gamma_q, gamma_k, pos_thw, dq, dk,
                              dgamma_q, dgamma_k, workspace, q_scale)


def abi_version() -> int:
    return int(load_library().h3attn_abi_version())

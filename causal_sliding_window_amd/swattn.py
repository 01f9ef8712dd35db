"""Thin Python binding of libswattn (argument marshalling only).

The entry points carry the C names of ``include/swattn.h`` and take torch tensors
that live on the GPU; every step of the computation runs in the HIP kernels of
``libswattn.so``.  Torch is used for device memory and streams only.  There is no
fallback: if the library is missing or fails to load, every call raises.

Convenience wrappers ``fwd``, ``bwd`` and ``decode`` allocate the outputs (and the
workspace) with torch and call the matching entry point for the input dtype; with
fewer K/V heads than query heads they call the grouped-query (``*_gqa``) entries.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswattn.so")

SWATTN_OK = 0
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float

_SIGS = {
    "swattn_status_string": ([_I], ctypes.c_char_p),
    "swattn_version": ([], _I),
    "swattn_fwd": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P], _I),
    "swattn_fwd_f32": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P], _I),
    "swattn_bwd_workspace_size": ([_I, _I, _I, _I], ctypes.c_size_t),
    "swattn_bwd": ([_P] * 9 + [_I] * 5 + [_F, _P, _P], _I),
    "swattn_bwd_f32": ([_P] * 9 + [_I] * 5 + [_F, _P, _P], _I),
    "swattn_bwd_preprocess": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "swattn_bwd_preprocess_f32": ([_P, _P, _P, _I, _I, _I, _I, _P], _I),
    "swattn_bwd_dkdv": ([_P] * 8 + [_I] * 5 + [_F, _P], _I),
    "swattn_bwd_dkdv_f32": ([_P] * 8 + [_I] * 5 + [_F, _P], _I),
    "swattn_bwd_dq": ([_P] * 8 + [_I] * 5 + [_F, _P], _I),
    "swattn_bwd_dq_f32": ([_P] * 8 + [_I] * 5 + [_F, _P], _I),
    "swattn_decode_workspace_size": ([_I] * 5, ctypes.c_size_t),
    "swattn_decode": ([_P] * 6 + [_I] * 5 + [_F, _P, _P], _I),
    "swattn_decode_f32": ([_P] * 6 + [_I] * 5 + [_F, _P, _P], _I),
    "swattn_decode_noalloc": ([_P] * 6 + [_I] * 5 + [_F, _P], _I),
    "swattn_fwd_gqa": ([_P] * 5 + [_I] * 6 + [_F, _P], _I),
    "swattn_bwd_gqa_workspace_size": ([_I] * 5, ctypes.c_size_t),
    "swattn_bwd_gqa": ([_P] * 9 + [_I] * 6 + [_F, _P, _P], _I),
    "swattn_decode_gqa": ([_P] * 6 + [_I] * 6 + [_F, _P, _P], _I),
    "swattn_prefill": ([_P] * 8 + [_I] * 7 + [_F, _P], _I),
    "swattn_qk_norm_rope": ([_P] * 5 + [_I] * 5 + [_F, _F, _P], _I),
    "swattn_qk_norm_rope_bwd": ([_P] * 7 + [_I] * 5 + [_F, _F, _P], _I),
    "swattn_fwd_rope": ([_P] * 7 + [_I] * 5 + [_F, _F, _F, _P], _I),
    "swattn_bwd_rope": ([_P] * 12 + [_I] * 5 + [_F, _F, _F, _P, _P], _I),
    "swattn_fwd_rope_gqa": ([_P] * 7 + [_I] * 6 + [_F, _F, _F, _P], _I),
    "swattn_bwd_rope_gqa": ([_P] * 12 + [_I] * 6 + [_F, _F, _F, _P, _P], _I),
    "swattn_probe_mfma": ([_P, _I, _I, _P], _I),
    "swattn_probe_read": ([_P, ctypes.c_size_t, _P, _I, _P], _I),
}


class SwattnError(RuntimeError):
    pass


def lib():
    """Load libswattn.so once (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SwattnError(
                f"{LIB_PATH} is missing: build it with `python -m causal_sliding_window_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
    return _lib


def status_string(code: int) -> str:
    return lib().swattn_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code != SWATTN_OK:
        raise SwattnError(f"{what} failed: {status_string(code)}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_tensor(t, name, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SwattnError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise SwattnError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SwattnError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise SwattnError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _kind(dtype):
    if dtype == torch.bfloat16:
        return ""
    if dtype == torch.float32:
        return "_f32"
    raise SwattnError(f"unsupported dtype {dtype}; use bfloat16 or float32")


# ----------------------------------------------------------------------------- C-named entries
def swattn_fwd(q, k, v, o, lse, window: int, scale: float, stream=None):
    """Forward into preallocated o [B,T,H,D] and lse [B,H,T] (float32)."""
    B, T, H, D = q.shape
    suf = _kind(q.dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _dev_tensor(t, n, q.dtype, (B, T, H, D))
    _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    fn = getattr(lib(), "swattn_fwd" + suf)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, T, D, int(window),
              float(scale), _stream(stream, q.device)), "swattn_fwd" + suf)


swattn_fwd_f32 = swattn_fwd


def swattn_bwd_workspace_size(B: int, H: int, T: int, D: int) -> int:
    return int(lib().swattn_bwd_workspace_size(B, H, T, D))


def swattn_bwd(q, k, v, o, do, lse, dq, dk, dv, window: int, scale: float, workspace,
               stream=None):
    """Backward into preallocated dq, dk, dv; ``workspace`` is a uint8 GPU tensor."""
    B, T, H, D = q.shape
    suf = _kind(q.dtype)
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk),
                 ("dv", dv)):
        _dev_tensor(t, n, q.dtype, (B, T, H, D))
    _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    _dev_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < swattn_bwd_workspace_size(B, H, T, D):
        raise SwattnError("workspace too small")
    fn = getattr(lib(), "swattn_bwd" + suf)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
              _ptr(dv), B, H, T, D, int(window), float(scale), _ptr(workspace),
              _stream(stream, q.device)), "swattn_bwd" + suf)


swattn_bwd_f32 = swattn_bwd


def _bwd_stage_checks(q, tensors, lse, workspace):
    B, T, H, D = q.shape
    for n, t in tensors:
        _dev_tensor(t, n, q.dtype, (B, T, H, D))
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    _dev_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < swattn_bwd_workspace_size(B, H, T, D):
        raise SwattnError("workspace too small")
    return B, T, H, D


def swattn_bwd_preprocess(o, do, workspace, stream=None):
    """delta = rowsum(dO * o) into the workspace (only needed to run dK/dV before dQ)."""
    B, T, H, D = _bwd_stage_checks(o, (("o", o), ("do", do)), None, workspace)
    fn = getattr(lib(), "swattn_bwd_preprocess" + _kind(o.dtype))
    _check(fn(_ptr(o), _ptr(do), _ptr(workspace), B, H, T, D, _stream(stream, o.device)),
           "swattn_bwd_preprocess")


def swattn_bwd_dkdv(q, k, v, do, lse, workspace, dk, dv, window: int, scale: float, stream=None):
    """dK, dV pass; reads delta from the workspace (written by swattn_bwd_dq or the
    preprocess)."""
    B, T, H, D = _bwd_stage_checks(q, (("q", q), ("k", k), ("v", v), ("do", do), ("dk", dk),
                                       ("dv", dv)), lse, workspace)
    fn = getattr(lib(), "swattn_bwd_dkdv" + _kind(q.dtype))
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(workspace), _ptr(dk), _ptr(dv),
              B, H, T, D, int(window), float(scale), _stream(stream, q.device)), "swattn_bwd_dkdv")


def swattn_bwd_dq(q, k, v, o, do, lse, workspace, dq, window: int, scale: float, stream=None):
    """dQ pass; also writes delta = rowsum(dO * o) into the workspace."""
    B, T, H, D = _bwd_stage_checks(q, (("q", q), ("k", k), ("v", v), ("o", o), ("do", do),
                                       ("dq", dq)), lse, workspace)
    fn = getattr(lib(), "swattn_bwd_dq" + _kind(q.dtype))
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(workspace), _ptr(dq),
              B, H, T, D, int(window), float(scale), _stream(stream, q.device)), "swattn_bwd_dq")


swattn_bwd_preprocess_f32 = swattn_bwd_preprocess
swattn_bwd_dkdv_f32 = swattn_bwd_dkdv
swattn_bwd_dq_f32 = swattn_bwd_dq


def swattn_decode_workspace_size(B: int, H: int, D: int, Tmax: int, window: int) -> int:
    return int(lib().swattn_decode_workspace_size(B, H, D, Tmax, int(window)))


def swattn_decode(q, k_cache, v_cache, seqlens, o, lse, window: int, scale: float, workspace,
                  stream=None):
    """Decode into preallocated o [B,H,D] (and lse [B,H] float32, or None)."""
    B, H, D = q.shape
    Tmax = k_cache.shape[1]
    suf = _kind(q.dtype)
    _dev_tensor(q, "q", q.dtype, (B, H, D))
    _dev_tensor(o, "o", q.dtype, (B, H, D))
    _dev_tensor(k_cache, "k_cache", q.dtype, (B, Tmax, H, D))
    _dev_tensor(v_cache, "v_cache", q.dtype, (B, Tmax, H, D))
    _dev_tensor(seqlens, "seqlens", torch.int32, (B,))
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32, (B, H))
    _dev_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < swattn_decode_workspace_size(B, H, D, Tmax, window):
        raise SwattnError("workspace too small")
    fn = getattr(lib(), "swattn_decode" + suf)
    _check(fn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse), B, H, D,
              Tmax, int(window), float(scale), _ptr(workspace), _stream(stream, q.device)),
           "swattn_decode" + suf)


swattn_decode_f32 = swattn_decode


def swattn_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, window: int, scale: float,
                          stream=None):
    """Allocation-free decode (bf16): as swattn_decode, with the library's own scratch
    array instead of a workspace (no device allocation anywhere in the call)."""
    B, H, D = q.shape
    Tmax = k_cache.shape[1]
    for n, t, shape in (("q", q, (B, H, D)), ("o", o, (B, H, D)),
                        ("k_cache", k_cache, (B, Tmax, H, D)),
                        ("v_cache", v_cache, (B, Tmax, H, D))):
        _dev_tensor(t, n, torch.bfloat16, shape)
    _dev_tensor(seqlens, "seqlens", torch.int32, (B,))
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32, (B, H))
    _check(lib().swattn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens),
                                       _ptr(o), _ptr(lse), B, H, D, Tmax, int(window),
                                       float(scale), _stream(stream, q.device)),
           "swattn_decode_noalloc")


# ----------------------------------------------------------------------------- measurement probes
def swattn_probe_mfma(out, workgroups: int, iters: int, stream=None):
    """Matrix-core rate probe: out float32 [workgroups * 256] (device); flops =
    workgroups * 4 * iters * 4 * 32768; every element of out becomes iters / 64."""
    _dev_tensor(out, "out", torch.float32, (workgroups * 256,))
    _check(lib().swattn_probe_mfma(_ptr(out), int(workgroups), int(iters),
                                   _stream(stream, out.device)), "swattn_probe_mfma")


def swattn_probe_read(src, out, workgroups: int, stream=None):
    """Streaming-read probe over the bytes of the contiguous device tensor src; out
    int32 [workgroups * 256] (device) receives per-thread XORs of the words read."""
    if not (src.is_cuda and src.is_contiguous()):
        raise SwattnError("src must be a contiguous device tensor")
    _dev_tensor(out, "out", torch.int32, (workgroups * 256,))
    _check(lib().swattn_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(out),
                                   int(workgroups), _stream(stream, src.device)),
           "swattn_probe_read")


# ----------------------------------------------------------------------------- grouped-query entries
def _groups(H, Hkv):
    if Hkv <= 0 or H % Hkv:
        raise SwattnError(f"{H} query heads cannot share {Hkv} K/V heads in equal groups")


def swattn_fwd_gqa(q, k, v, o, lse, window: int, scale: float, stream=None):
    """Grouped-query forward (bf16): q, o [B,T,H,D]; k, v [B,T,Hkv,D]; lse [B,H,T]."""
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    _groups(H, Hkv)
    for n, t, h in (("q", q, H), ("k", k, Hkv), ("v", v, Hkv), ("o", o, H)):
        _dev_tensor(t, n, torch.bfloat16, (B, T, h, D))
    _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    _check(lib().swattn_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, T, D,
                                int(window), float(scale), _stream(stream, q.device)),
           "swattn_fwd_gqa")


def swattn_bwd_gqa_workspace_size(B: int, H: int, Hkv: int, T: int, D: int) -> int:
    return int(lib().swattn_bwd_gqa_workspace_size(B, H, Hkv, T, D))


def swattn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, window: int, scale: float, workspace,
                   stream=None):
    """Grouped-query backward (bf16): dq [B,T,H,D]; dk, dv [B,T,Hkv,D] (sums over each
    K/V head's query heads)."""
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    _groups(H, Hkv)
    for n, t, h in (("q", q, H), ("k", k, Hkv), ("v", v, Hkv), ("o", o, H), ("do", do, H),
                    ("dq", dq, H), ("dk", dk, Hkv), ("dv", dv, Hkv)):
        _dev_tensor(t, n, torch.bfloat16, (B, T, h, D))
    _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    _dev_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < swattn_bwd_gqa_workspace_size(B, H, Hkv, T,
                                                                                     D):
        raise SwattnError("workspace too small")
    _check(lib().swattn_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                _ptr(dk), _ptr(dv), B, H, Hkv, T, D, int(window), float(scale),
                                _ptr(workspace), _stream(stream, q.device)), "swattn_bwd_gqa")


def swattn_decode_gqa(q, k_cache, v_cache, seqlens, o, lse, window: int, scale: float,
                      workspace, stream=None):
    """Grouped-query decode (bf16): q, o [B,H,D]; k_cache, v_cache [B,Tmax,Hkv,D]."""
    B, H, D = q.shape
    Tmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    _groups(H, Hkv)
    _dev_tensor(q, "q", torch.bfloat16, (B, H, D))
    _dev_tensor(o, "o", torch.bfloat16, (B, H, D))
    _dev_tensor(k_cache, "k_cache", torch.bfloat16, (B, Tmax, Hkv, D))
    _dev_tensor(v_cache, "v_cache", torch.bfloat16, (B, Tmax, Hkv, D))
    _dev_tensor(seqlens, "seqlens", torch.int32, (B,))
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32, (B, H))
    _dev_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < swattn_decode_workspace_size(B, H, D, Tmax, window):
        raise SwattnError("workspace too small")
    _check(lib().swattn_decode_gqa(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o),
                                   _ptr(lse), B, H, Hkv, D, Tmax, int(window), float(scale),
                                   _ptr(workspace), _stream(stream, q.device)),
           "swattn_decode_gqa")


def swattn_prefill(q, k_new, v_new, k_cache, v_cache, seqlens, o, lse, window: int,
                   scale: float, stream=None):
    """Chunked prefill (bf16): appends k_new, v_new [B,Tq,Hkv,D] to the caches [B,Tmax,Hkv,D]
    at seqlens (clamped to [0, Tmax - Tq]) and attends q [B,Tq,H,D] against them into o
    (and lse [B,H,Tq] unless None)."""
    B, Tq, H, D = q.shape
    Tmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    _groups(H, Hkv)
    for n, t, shape in (("q", q, (B, Tq, H, D)), ("o", o, (B, Tq, H, D)),
                        ("k_new", k_new, (B, Tq, Hkv, D)), ("v_new", v_new, (B, Tq, Hkv, D)),
                        ("k_cache", k_cache, (B, Tmax, Hkv, D)),
                        ("v_cache", v_cache, (B, Tmax, Hkv, D))):
        _dev_tensor(t, n, torch.bfloat16, shape)
    _dev_tensor(seqlens, "seqlens", torch.int32, (B,))
    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32, (B, H, Tq))
    _check(lib().swattn_prefill(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                _ptr(seqlens), _ptr(o), _ptr(lse), B, H, Hkv, Tq, D, Tmax,
                                int(window), float(scale), _stream(stream, q.device)),
           "swattn_prefill")


def _prologue_shapes(q, k, pos_offset, tensors):
    """Shapes of a prologue call; q or k may be None (that side absent: H or Hkv = 0)."""
    ref = q if q is not None else k
    if ref is None:
        raise SwattnError("the prologue needs q or k")
    B, T, _, D = ref.shape
    H = 0 if q is None else q.shape[2]
    Hkv = 0 if k is None else k.shape[2]
    for n, t in tensors:
        is_q = n.startswith(("q", "dq"))
        if (H if is_q else Hkv) == 0:
            if t is not None:
                raise SwattnError(f"{n} given for an absent side")
            continue
        _dev_tensor(t, n, torch.bfloat16, (B, T, H, D) if is_q else (B, T, Hkv, D))
    if pos_offset is not None:
        _dev_tensor(pos_offset, "pos_offset", torch.int32, (B,))
    return B, T, H, Hkv, D


def swattn_qk_norm_rope(q, k, q_out, k_out, pos_offset=None, base: float = 10000.0,
                        eps: float = 1e-6, stream=None):
    """QK-norm + rotary prologue (bf16): q [B,T,H,D], k [B,T,Hkv,D] -> q_out, k_out;
    token t of sequence b at position max(pos_offset[b], 0) + t (t without offsets)."""
    B, T, H, Hkv, D = _prologue_shapes(q, k, pos_offset, (("q", q), ("k", k), ("q_out", q_out),
                                                          ("k_out", k_out)))
    _check(lib().swattn_qk_norm_rope(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(pos_offset),
                                     B, T, H, Hkv, D, float(base), float(eps),
                                     _stream(stream, (q if q is not None else k).device)),
           "swattn_qk_norm_rope")


def swattn_qk_norm_rope_bwd(q, k, dq_out, dk_out, dq, dk, pos_offset=None,
                            base: float = 10000.0, eps: float = 1e-6, stream=None):
    """Backward of the prologue: raw q, k and the gradients of its outputs -> dq, dk."""
    B, T, H, Hkv, D = _prologue_shapes(q, k, pos_offset, (
        ("q", q), ("k", k), ("dq_out", dq_out), ("dk_out", dk_out), ("dq", dq), ("dk", dk)))
    _check(lib().swattn_qk_norm_rope_bwd(_ptr(q), _ptr(k), _ptr(dq_out), _ptr(dk_out), _ptr(dq),
                                         _ptr(dk), _ptr(pos_offset), B, T, H, Hkv, D, float(base),
                                         float(eps),
                                         _stream(stream, (q if q is not None else k).device)),
           "swattn_qk_norm_rope_bwd")


def swattn_fwd_rope(q, k_rope, v, o, lse, q_rope, window: int, scale: float, pos_offset=None,
                    base: float = 10000.0, eps: float = 1e-6, stream=None):
    """Forward with the QK-norm + rotary prologue fused into the query load (bf16, H == Hkv):
    raw q, transformed k_rope; q_rope (or None) receives the transformed queries."""
    B, T, H, D = q.shape
    for n, t in (("q", q), ("k_rope", k_rope), ("v", v), ("o", o)):
        _dev_tensor(t, n, torch.bfloat16, (B, T, H, D))
    if q_rope is not None:
        _dev_tensor(q_rope, "q_rope", torch.bfloat16, (B, T, H, D))
    _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    if pos_offset is not None:
        _dev_tensor(pos_offset, "pos_offset", torch.int32, (B,))
    _check(lib().swattn_fwd_rope(_ptr(q), _ptr(k_rope), _ptr(v), _ptr(o), _ptr(lse), _ptr(q_rope),
                                 _ptr(pos_offset), B, H, T, D, int(window), float(scale),
                                 float(base), float(eps), _stream(stream, q.device)),
           "swattn_fwd_rope")


def swattn_bwd_rope(q, k, q_rope, k_rope, v, o, do, lse, dq, dk, dv, window: int, scale: float,
                    workspace, pos_offset=None, base: float = 10000.0, eps: float = 1e-6,
                    stream=None):
    """Backward through attention and the fused prologue (bf16, H == Hkv): dq, dk with
    respect to the raw q, k."""
    B, T, H, D = q.shape
    for n, t in (("q", q), ("k", k), ("q_rope", q_rope), ("k_rope", k_rope), ("v", v), ("o", o),
                 ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _dev_tensor(t, n, torch.bfloat16, (B, T, H, D))
    _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    if pos_offset is not None:
        _dev_tensor(pos_offset, "pos_offset", torch.int32, (B,))
    _dev_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < swattn_bwd_workspace_size(B, H, T, D):
        raise SwattnError("workspace too small")
    _check(lib().swattn_bwd_rope(_ptr(q), _ptr(k), _ptr(q_rope), _ptr(k_rope), _ptr(v), _ptr(o),
                                 _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(pos_offset), B, H, T, D, int(window), float(scale),
                                 float(base), float(eps), _ptr(workspace),
                                 _stream(stream, q.device)), "swattn_bwd_rope")


def swattn_fwd_rope_gqa(q, k_rope, v, o, lse, q_rope, window: int, scale: float,
                        pos_offset=None, base: float = 10000.0, eps: float = 1e-6, stream=None):
    """swattn_fwd_rope with K/V head groups: k_rope, v [B,T,Hkv,D]."""
    B, T, H, D = q.shape
    Hkv = k_rope.shape[2]
    _groups(H, Hkv)
    for n, t in (("q", q), ("o", o)):
        _dev_tensor(t, n, torch.bfloat16, (B, T, H, D))
    for n, t in (("k_rope", k_rope), ("v", v)):
        _dev_tensor(t, n, torch.bfloat16, (B, T, Hkv, D))
    if q_rope is not None:
        _dev_tensor(q_rope, "q_rope", torch.bfloat16, (B, T, H, D))
    _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    if pos_offset is not None:
        _dev_tensor(pos_offset, "pos_offset", torch.int32, (B,))
    _check(lib().swattn_fwd_rope_gqa(_ptr(q), _ptr(k_rope), _ptr(v), _ptr(o), _ptr(lse),
                                     _ptr(q_rope), _ptr(pos_offset), B, H, Hkv, T, D, int(window),
                                     float(scale), float(base), float(eps),
                                     _stream(stream, q.device)), "swattn_fwd_rope_gqa")


def swattn_bwd_rope_gqa(q, k, q_rope, k_rope, v, o, do, lse, dq, dk, dv, window: int,
                        scale: float, workspace, pos_offset=None, base: float = 10000.0,
                        eps: float = 1e-6, stream=None):
    """swattn_bwd_rope with K/V head groups: k, k_rope, v, dk, dv [B,T,Hkv,D]."""
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    _groups(H, Hkv)
    for n, t in (("q", q), ("q_rope", q_rope), ("o", o), ("do", do), ("dq", dq)):
        _dev_tensor(t, n, torch.bfloat16, (B, T, H, D))
    for n, t in (("k", k), ("k_rope", k_rope), ("v", v), ("dk", dk), ("dv", dv)):
        _dev_tensor(t, n, torch.bfloat16, (B, T, Hkv, D))
    _dev_tensor(lse, "lse", torch.float32, (B, H, T))
    if pos_offset is not None:
        _dev_tensor(pos_offset, "pos_offset", torch.int32, (B,))
    _dev_tensor(workspace, "workspace")
    if workspace.numel() * workspace.element_size() < swattn_bwd_gqa_workspace_size(B, H, Hkv, T,
                                                                                   D):
        raise SwattnError("workspace too small")
    _check(lib().swattn_bwd_rope_gqa(_ptr(q), _ptr(k), _ptr(q_rope), _ptr(k_rope), _ptr(v),
                                     _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                     _ptr(pos_offset), B, H, Hkv, T, D, int(window), float(scale),
                                     float(base), float(eps), _ptr(workspace),
                                     _stream(stream, q.device)), "swattn_bwd_rope_gqa")


# ----------------------------------------------------------------------------- allocating wrappers
def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def fwd(q, k, v, window: int = -1, scale: float | None = None, stream=None):
    B, T, H, D = q.shape
    scale = default_scale(D) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device)
    if k.shape[2] != H:
        swattn_fwd_gqa(q, k, v, o, lse, window, scale, stream)
    else:
        swattn_fwd(q, k, v, o, lse, window, scale, stream)
    return o, lse


def bwd(q, k, v, o, do, lse, window: int = -1, scale: float | None = None, stream=None,
        workspace=None):
    B, T, H, D = q.shape
    scale = default_scale(D) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    Hkv = k.shape[2]
    if workspace is None:
        workspace = torch.empty(swattn_bwd_gqa_workspace_size(B, H, Hkv, T, D), dtype=torch.uint8,
                                device=q.device)
    if Hkv != H:
        swattn_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, window, scale, workspace, stream)
    else:
        swattn_bwd(q, k, v, o, do, lse, dq, dk, dv, window, scale, workspace, stream)
    return dq, dk, dv


def prefill(q, k_new, v_new, k_cache, v_cache, seqlens, window: int = -1,
            scale: float | None = None, stream=None, with_lse: bool = True):
    """Appends the chunk to the caches in place and returns (o, lse) of its queries."""
    B, Tq, H, D = q.shape
    scale = default_scale(D) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device) if with_lse else None
    swattn_prefill(q, k_new, v_new, k_cache, v_cache, seqlens, o, lse, window, scale, stream)
    return o, lse


def decode(q, k_cache, v_cache, seqlens, window: int = -1, scale: float | None = None,
           stream=None, workspace=None, with_lse: bool = True):
    B, H, D = q.shape
    Tmax = k_cache.shape[1]
    scale = default_scale(D) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if with_lse else None
    if workspace is None:
        workspace = torch.empty(swattn_decode_workspace_size(B, H, D, Tmax, window),
                                dtype=torch.uint8, device=q.device)
    if k_cache.shape[2] != H:
        swattn_decode_gqa(q, k_cache, v_cache, seqlens, o, lse, window, scale, workspace, stream)
    else:
        swattn_decode(q, k_cache, v_cache, seqlens, o, lse, window, scale, workspace, stream)
    return o, lse


def qk_norm_rope(q, k, pos_offset=None, base: float = 10000.0, eps: float = 1e-6, stream=None):
    """Returns (q', k'): every head vector RMS-normalised and rotated by its position."""
    q_out, k_out = torch.empty_like(q), torch.empty_like(k)
    swattn_qk_norm_rope(q, k, q_out, k_out, pos_offset, base, eps, stream)
    return q_out, k_out


def qk_norm_rope_bwd(q, k, dq_out, dk_out, pos_offset=None, base: float = 10000.0,
                     eps: float = 1e-6, stream=None):
    """Returns (dq, dk) for the raw q, k given the gradients of (q', k')."""
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    swattn_qk_norm_rope_bwd(q, k, dq_out, dk_out, dq, dk, pos_offset, base, eps, stream)
    return dq, dk

"""Python binding of libfa.so (the C ABI in include/fa.h).

Argument marshalling only: the functions below check that the torch tensors
have the layout the C ABI documents, pass raw device pointers and the
caller's current HIP stream to ``fa_fwd`` / ``fa_bwd``, and raise
``FAError`` on a non-OK status.  Every step of the computation runs in the
HIP kernels; there is no fallback.  If libfa.so is missing or cannot be
loaded, the first call raises.

torch is imported before the library is loaded so that libfa.so binds to the
HIP runtime torch has already mapped (both carry the soname libamdhip64.so.7).
"""

from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fa.h")

FA_BF16, FA_FP32 = 0, 1
MASK_BLOCK = 128

STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEAD_DIM",
    4: "FA_ERR_DTYPE", 5: "FA_ERR_ALIGN", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_LAUNCH",
    8: "FA_ERR_ARG", 9: "FA_ERR_ALIAS", 10: "FA_ERR_SCRATCH",
}
STATIC_SCRATCH_BYTES = 4194304     # FA_STATIC_SCRATCH_BYTES of include/fa.h


class FAError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so (once) and declare its C signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"libfa.so not found at {path}; build it first "
                "(python -m io_aware_exact_09_amd.build)")
        lib = ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
        lib.fa_fwd.restype = i
        lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i]
        lib.fa_fwd_workspace_bytes.argtypes = [i, i, i, i]
        lib.fa_fwd_workspace_bytes.restype = sz
        lib.fa_fwd_ws.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
        lib.fa_fwd_ws.restype = i
        lib.fa_bwd_splits.argtypes = [i, i, i, i, i, i, ctypes.POINTER(ctypes.c_int),
                                      ctypes.POINTER(ctypes.c_int)]
        lib.fa_bwd_splits.restype = ctypes.c_int
        lib.fa_bwd_workspace_bytes.restype = sz
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i,
                               vp, sz, vp]
        lib.fa_bwd.restype = i
        lib.fa_bwd_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp,
                                      i, vp]
        lib.fa_bwd_static.restype = i
        lib.fa_bwd_preprocess.argtypes = [vp, vp, i, i, i, i, i, vp, sz, vp]
        lib.fa_bwd_preprocess.restype = i
        lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz,
                                    vp]
        lib.fa_bwd_dkdv.restype = i
        lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
        lib.fa_bwd_dq.restype = i
        lib.fa_bwd_dq_and_d.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i,
                                        vp, sz, vp]
        lib.fa_bwd_dq_and_d.restype = i
        u64 = ctypes.c_ulonglong
        lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, f, u64, i, vp]
        lib.fa_fwd_dropout.restype = i
        lib.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp,
                                       f, u64, i, vp, sz, vp]
        lib.fa_bwd_dropout.restype = i
        lib.fa_bwd_gqa_workspace_bytes.argtypes = [i, i, i, i, i]
        lib.fa_bwd_gqa_workspace_bytes.restype = sz
        lib.fa_fwd_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp]
        lib.fa_fwd_gqa.restype = i
        lib.fa_bwd_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp,
                                   i, vp, sz, vp]
        lib.fa_bwd_gqa.restype = i
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp]
        lib.fa_fwd_fp8.restype = i
        lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, i, vp, sz,
                                  vp]
        lib.fa_decode.restype = i
        lib.fa_decode_num_splits.argtypes = [i] * 7
        lib.fa_decode_num_splits.restype = i
        lib.fa_decode_workspace_bytes.argtypes = [i] * 7
        lib.fa_decode_workspace_bytes.restype = sz
        lib.fa_status_str.argtypes = [i]
        lib.fa_status_str.restype = ctypes.c_char_p
        _lib = lib
        return lib


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/fa.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)


def status_str(status: int) -> str:
    return load_library().fa_status_str(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise FAError(status, where, status_str(status))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensors(ref: torch.Tensor, named: dict):
    if ref.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    for name, t in named.items():
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _scratch(nbytes: int, ref: torch.Tensor, stream=None) -> torch.Tensor:
    """Device scratch of ``nbytes`` bytes for one call, allocated by torch's
    caching allocator on the current stream.  When the call is enqueued on
    another ``stream``, the block is also recorded as in use by that stream,
    so the allocator does not hand it to a later allocation until the
    kernels reading and writing it there have finished."""
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=ref.device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, H, N, d))


def fa_bwd_splits(B: int, Hq: int, Hkv: int, N: int, d: int, dtype: str) -> tuple[int, int]:
    """(dK/dV split, dQ split) that fa_bwd / fa_bwd_gqa / fa_bwd_dropout use
    for this shape with a workspace of the preferred size."""
    kv, q = ctypes.c_int(0), ctypes.c_int(0)
    code = {"bf16": 0, "fp32": 1}[dtype]
    _check(load_library().fa_bwd_splits(B, Hq, Hkv, N, d, code, ctypes.byref(kv),
                                        ctypes.byref(q)), "fa_bwd_splits")
    return kv.value, q.value


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool = False, block_mask=None,
           stream=None) -> None:
    """Enqueue the forward on ``stream`` (default: torch's current stream).

    q, k, v, o: [B,H,N,d] bf16 or fp32 device tensors; lse: [B,H,N] fp32;
    block_mask: None or a uint8 [ceil(N/128)]^2 device tensor.
    """
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, lse=lse))
    B, H, N, d = q.shape
    if block_mask is not None:
        _check_tensors(q, dict(block_mask=block_mask))
        if block_mask.dtype != torch.uint8:
            raise TypeError("block_mask must be uint8")
    st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                    int(bool(causal)), _ptr(block_mask), _dtype_code(q), _stream(stream))
    _check(st, "fa_fwd")


def fa_fwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_fwd_workspace_bytes(B, H, N, d))


def fa_fwd_ws(q, k, v, o, lse, scale: float, causal: bool = False, block_mask=None,
              workspace=None, stream=None) -> None:
    """fa_fwd with a workspace, which lets shapes that fill few compute units
    run split (``workspace``: a device tensor of fa_fwd_workspace_bytes(B, H,
    N, d) bytes, allocated here if None; None and a size of 0: plain fa_fwd)."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, lse=lse))
    B, H, N, d = q.shape
    if block_mask is not None:
        _check_tensors(q, dict(block_mask=block_mask))
        if block_mask.dtype != torch.uint8:
            raise TypeError("block_mask must be uint8")
    if workspace is None:
        need = fa_fwd_workspace_bytes(B, H, N, d)
        workspace = _scratch(need, q, stream) if need else None
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.fa_fwd_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                       int(bool(causal)), _ptr(block_mask), _dtype_code(q), _ptr(workspace),
                       wbytes, _stream(stream))
    _check(st, "fa_fwd_ws")


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False,
           block_mask=None, workspace=None, stream=None) -> None:
    """Enqueue the backward.  ``workspace``: a device tensor of at least
    fa_bwd_workspace_bytes(B, H, N, d) bytes (allocated here if None)."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv))
    B, H, N, d = q.shape
    if workspace is None:
        workspace = _scratch(fa_bwd_workspace_bytes(B, H, N, d), q, stream)
    wbytes = workspace.numel() * workspace.element_size()
    if block_mask is not None:
        _check_tensors(q, dict(block_mask=block_mask))
        if block_mask.dtype != torch.uint8:
            raise TypeError("block_mask must be uint8")
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                    _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                    _ptr(block_mask), _dtype_code(q), _ptr(workspace), wbytes,
                    _stream(stream))
    _check(st, "fa_bwd")


def fa_bwd_static(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False,
                  block_mask=None, stream=None) -> None:
    """fa_bwd without a workspace: D goes to the library's static device
    scratch, so the call allocates nothing (here or in the library).  Needs
    4 * B * H * N <= STATIC_SCRATCH_BYTES; calls that overlap on one GPU race
    on the shared scratch."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv))
    _mask_ok(q, block_mask)
    B, H, N, d = q.shape
    st = lib.fa_bwd_static(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                           _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                           _ptr(block_mask), _dtype_code(q), _stream(stream))
    _check(st, "fa_bwd_static")


def fa_fwd_dropout(q, k, v, o, lse, scale: float, dropout_p: float, seed: int,
                   causal: bool = False, block_mask=None, stream=None) -> None:
    """fa_fwd with dropout on the probabilities (keep probability 1 - p; the
    keep mask is regenerated from ``seed`` by fa_bwd_dropout)."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, lse=lse))
    _mask_ok(q, block_mask)
    B, H, N, d = q.shape
    st = lib.fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                            float(scale), int(bool(causal)), _ptr(block_mask), float(dropout_p),
                            int(seed) & (2 ** 64 - 1), _dtype_code(q), _stream(stream))
    _check(st, "fa_fwd_dropout")


def fa_bwd_dropout(q, k, v, o, do, lse, dq, dk, dv, scale: float, dropout_p: float, seed: int,
                   causal: bool = False, block_mask=None, workspace=None, stream=None) -> None:
    """fa_bwd for outputs of fa_fwd_dropout (same dropout_p and seed)."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv))
    _mask_ok(q, block_mask)
    B, H, N, d = q.shape
    if workspace is None:
        workspace = _scratch(fa_bwd_workspace_bytes(B, H, N, d), q, stream)
    st = lib.fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                            _ptr(block_mask), float(dropout_p), int(seed) & (2 ** 64 - 1),
                            _dtype_code(q), _ptr(workspace), _nbytes(workspace),
                            _stream(stream))
    _check(st, "fa_bwd_dropout")


def _mask_ok(q, block_mask):
    if block_mask is not None:
        _check_tensors(q, dict(block_mask=block_mask))
        if block_mask.dtype != torch.uint8:
            raise TypeError("block_mask must be uint8")


def _nbytes(t):
    return t.numel() * t.element_size()


def fa_bwd_preprocess(o, do, workspace, stream=None) -> None:
    """D_i = rowsum(dO * O) into ``workspace`` (first phase of fa_bwd)."""
    lib = load_library()
    _check_tensors(o, dict(o=o, do=do, workspace=workspace))
    B, H, N, d = o.shape
    st = lib.fa_bwd_preprocess(_ptr(o), _ptr(do), B, H, N, d, _dtype_code(o), _ptr(workspace),
                               _nbytes(workspace), _stream(stream))
    _check(st, "fa_bwd_preprocess")


def fa_bwd_dkdv(q, k, v, do, lse, dk, dv, scale, causal=False, block_mask=None,
                workspace=None, stream=None) -> None:
    """dK, dV pass (second phase of fa_bwd); ``workspace`` holds D."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, do=do, lse=lse, dk=dk, dv=dv, workspace=workspace))
    _mask_ok(q, block_mask)
    B, H, N, d = q.shape
    st = lib.fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dk), _ptr(dv),
                         B, H, N, d, float(scale), int(bool(causal)), _ptr(block_mask),
                         _dtype_code(q), _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, do, lse, dq, scale, causal=False, block_mask=None, workspace=None,
              stream=None) -> None:
    """dQ pass (third phase of fa_bwd); ``workspace`` holds D."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, do=do, lse=lse, dq=dq, workspace=workspace))
    _mask_ok(q, block_mask)
    B, H, N, d = q.shape
    st = lib.fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dq), B, H, N, d,
                       float(scale), int(bool(causal)), _ptr(block_mask), _dtype_code(q),
                       _ptr(workspace), _nbytes(workspace), _stream(stream))
    _check(st, "fa_bwd_dq")


def fa_bwd_dq_and_d(q, k, v, o, do, lse, dq, scale, causal=False, block_mask=None,
                    workspace=None, stream=None) -> None:
    """dQ pass that forms D from O and dO and writes it to ``workspace``
    (fa_bwd is this, then fa_bwd_dkdv)."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, workspace=workspace))
    _mask_ok(q, block_mask)
    B, H, N, d = q.shape
    st = lib.fa_bwd_dq_and_d(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                             B, H, N, d, float(scale), int(bool(causal)), _ptr(block_mask),
                             _dtype_code(q), _ptr(workspace), _nbytes(workspace),
                             _stream(stream))
    _check(st, "fa_bwd_dq_and_d")


def fa_bwd_gqa_workspace_bytes(B: int, Hq: int, Hkv: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_gqa_workspace_bytes(B, Hq, Hkv, N, d))


def fa_fwd_gqa(q, k, v, o, lse, scale: float, causal: bool = False, block_mask=None,
               stream=None) -> None:
    """Forward with grouped key/value heads: q, o [B,Hq,N,d]; k, v [B,Hkv,N,d]."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, lse=lse))
    _mask_ok(q, block_mask)
    B, Hq, N, d = q.shape
    st = lib.fa_fwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, k.shape[1], N, d,
                        float(scale), int(bool(causal)), _ptr(block_mask), _dtype_code(q),
                        _stream(stream))
    _check(st, "fa_fwd_gqa")


def fa_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool = False,
               block_mask=None, workspace=None, stream=None) -> None:
    """Backward with grouped key/value heads (dk, dv: [B,Hkv,N,d])."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, do=do, lse=lse, dq=dq, dk=dk, dv=dv))
    _mask_ok(q, block_mask)
    B, Hq, N, d = q.shape
    if workspace is None:
        need = int(lib.fa_bwd_gqa_workspace_bytes(B, Hq, k.shape[1], N, d))
        workspace = _scratch(need, q, stream)
    st = lib.fa_bwd_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                        _ptr(dk), _ptr(dv), B, Hq, k.shape[1], N, d, float(scale),
                        int(bool(causal)), _ptr(block_mask), _dtype_code(q), _ptr(workspace),
                        _nbytes(workspace), _stream(stream))
    _check(st, "fa_bwd_gqa")


def fa_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, o, lse, scale: float,
               causal: bool = False, block_mask=None, stream=None) -> None:
    """FP8 (E4M3) forward: q8, k8 uint8 [B,H,N,d]; vt8 uint8 [B,H,d,N] (V
    transposed); q_scale, k_scale fp32 [B,H,ceil(N/128)]; v_scale fp32 [B,H];
    o bf16 [B,H,N,d]; lse fp32 [B,H,N]."""
    lib = load_library()
    _check_tensors(q8, dict(q8=q8, k8=k8, vt8=vt8, q_scale=q_scale, k_scale=k_scale,
                            v_scale=v_scale, o=o, lse=lse))
    _mask_ok(q8, block_mask)
    for name, t in (("q8", q8), ("k8", k8), ("vt8", vt8)):
        if t.dtype != torch.uint8:
            raise TypeError(f"{name} must hold uint8 E4M3 codes")
    if o.dtype != torch.bfloat16:
        raise TypeError("o must be bfloat16")
    B, H, N, d = q8.shape
    st = lib.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(q_scale), _ptr(k_scale),
                        _ptr(v_scale), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                        int(bool(causal)), _ptr(block_mask), _stream(stream))
    _check(st, "fa_fwd_fp8")


def fa_decode_num_splits(B, Hq, Hkv, Nq, Nkv, d, num_splits=0) -> int:
    """Key chunks fa_decode uses for these sizes (0 for rejected sizes)."""
    return int(load_library().fa_decode_num_splits(B, Hq, Hkv, Nq, Nkv, d, num_splits))


def fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, num_splits=0) -> int:
    return int(load_library().fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, num_splits))


def fa_decode(q, k, v, o, lse, scale: float, seqlens=None, causal: bool = False,
              num_splits: int = 0, workspace=None, stream=None) -> None:
    """Enqueue decode attention: q, o [B,Hq,Nq,d]; k, v (the cache)
    [B,Hkv,Nkv,d]; lse [B,Hq,Nq] fp32; seqlens None or an int32 device tensor
    [B].  ``workspace`` is allocated here if None and needed."""
    lib = load_library()
    _check_tensors(q, dict(q=q, k=k, v=v, o=o, lse=lse))
    B, Hq, Nq, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    if seqlens is not None:
        _check_tensors(q, dict(seqlens=seqlens))
        if seqlens.dtype != torch.int32:
            raise TypeError("seqlens must be int32")
    need = fa_decode_workspace_bytes(B, Hq, Hkv, Nq, Nkv, d, num_splits)
    if workspace is None and need:
        workspace = _scratch(need, q, stream)
    wbytes = 0 if workspace is None else _nbytes(workspace)
    st = lib.fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv,
                       Nq, Nkv, d, float(scale), int(bool(causal)), int(num_splits),
                       _dtype_code(q), _ptr(workspace), wbytes, _stream(stream))
    _check(st, "fa_decode")


# Convenience wrappers that allocate outputs with torch (memory plumbing only).
# The outputs come from torch's current stream; when the work is enqueued on
# another ``stream`` they are recorded as in use there too (see _scratch).

def _mark(stream, *ts):
    if stream is not None:
        for t in ts:
            t.record_stream(stream)


def decode(q, k, v, scale: float, seqlens=None, causal: bool = False, num_splits: int = 0,
           workspace=None, stream=None):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _mark(stream, o, lse)
    fa_decode(q, k, v, o, lse, scale, seqlens, causal, num_splits, workspace, stream)
    return o, lse


def forward(q, k, v, scale: float, causal: bool = False, block_mask=None, stream=None):
    """O, LSE through fa_fwd_ws (so shapes that fill few compute units run split)."""
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _mark(stream, o, lse)
    fa_fwd_ws(q, k, v, o, lse, scale, causal, block_mask, None, stream)
    return o, lse


def backward(q, k, v, o, do, lse, scale: float, causal: bool = False, block_mask=None,
             workspace=None, stream=None):
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _mark(stream, dq, dk, dv)
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale, causal, block_mask, workspace, stream)
    return dq, dk, dv

"""Exact, IO-aware tiled attention for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libfa.so`` (declared in
``include/fa.h``).  Every step of the computation runs in the library's HIP
kernels; this module only checks tensors, allocates outputs with torch, and
passes raw device pointers plus torch's current HIP stream.  There is no CPU
fallback: if the library is missing, importing the binding's functions raises.

Functions take [B, H, N, d] contiguous CUDA (HIP) tensors of one dtype
(float32, float16 or bfloat16) and follow the semantics in ``include/fa.h``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
DEBUG_SYNC_LIB_PATH = os.path.join(_PKG, "libfa_debugsync.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_WORKSPACE = -3
FA_ERR_HIP = -4

SYMBOLS = ("fa_forward", "fa_forward_gqa", "fa_forward_blockmap", "fa_backward",
           "fa_backward_noalloc",
           "fa_backward_gqa", "fa_backward_blockmap",
           "fa_backward_stage", "fa_backward_workspace_size", "fa_backward_gqa_workspace_size",
           "fa_decode", "fa_decode_num_splits",
           "fa_decode_workspace_size", "fa_decode_stage", "fa_tile_config", "fa_strerror",
           "fa_last_error", "fa_fp8_quantize_rows", "fa_forward_fp8")

BWD_PREPROCESS, BWD_DKDV, BWD_DQ = 0, 1, 2
DEC_SPLIT, DEC_COMBINE = 0, 1


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so and declare its signatures (raises if it is not built).  The
    first library loaded serves every call of this module."""
    global _lib
    if _lib is None:
        _lib = open_library(path)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Load a build of the C ABI at `path` (e.g. the race-check variant
    libfa_debugsync.so) with its signatures declared, without making it the
    module's library."""
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m exact_io_aware_forward_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_forward.restype = i
    lib.fa_forward_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_forward_gqa.restype = i
    lib.fa_backward_gqa.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i,
                                    vp, sz, vp]
    lib.fa_backward_gqa.restype = i
    lib.fa_forward_blockmap.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp]
    lib.fa_forward_blockmap.restype = i
    lib.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_backward.restype = i
    lib.fa_backward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                                        vp]
    lib.fa_backward_noalloc.restype = i
    lib.fa_backward_blockmap.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                                         vp, sz, vp, vp, vp]
    lib.fa_backward_blockmap.restype = i
    lib.fa_backward_stage.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i,
                                      vp, sz, vp]
    lib.fa_backward_stage.restype = i
    lib.fa_backward_workspace_size.argtypes = [i, i, i, i]
    lib.fa_backward_workspace_size.restype = sz
    lib.fa_backward_gqa_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_backward_gqa_workspace_size.restype = sz
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_decode.restype = i
    lib.fa_decode_stage.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, sz,
                                    vp]
    lib.fa_decode_stage.restype = i
    lib.fa_decode_num_splits.argtypes = [i, i, i, i, i, i]
    lib.fa_decode_num_splits.restype = i
    lib.fa_decode_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_decode_workspace_size.restype = sz
    lib.fa_tile_config.argtypes = [i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.fa_tile_config.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_fp8_quantize_rows.argtypes = [vp, ctypes.c_longlong, i, i, vp, vp, vp, vp]
    lib.fa_fp8_quantize_rows.restype = i
    lib.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.fa_forward_fp8.restype = i
    return lib


def _check(status: int) -> None:
    if status != FA_OK:
        lib = load_library()
        detail = lib.fa_last_error().decode() or lib.fa_strerror(status).decode()
        raise FAError(status, detail)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(q: torch.Tensor, *others: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    for t in (q, *others):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("all tensors must share shape, dtype and device")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous GPU tensors")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return q.shape


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def tile_config(kernel_id: int, d: int, dtype: torch.dtype) -> tuple[int, int]:
    """(Br, Bc) of kernel 0 = forward with the causal mask, 1 = dK/dV, 2 = dQ,
    3 = forward without the causal mask."""
    lib = load_library()
    br, bc = ctypes.c_int(), ctypes.c_int()
    _check(lib.fa_tile_config(kernel_id, d, _DTYPE_CODE[dtype], ctypes.byref(br), ctypes.byref(bc)))
    return br.value, bc.value


def _kv_heads(q, k, v) -> int:
    """Key/value head count: k, v are [B, Hkv, N, d] with Hkv dividing q's H."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    _shape(k, v)
    if (k.shape[0], k.shape[2], k.shape[3]) != (q.shape[0], q.shape[2], q.shape[3]) \
            or q.shape[1] % k.shape[1]:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing q's head count")
    return k.shape[1]


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """O, LSE = attention(q, k, v).  O has q's dtype, LSE is float32 [B, H, N].
    k, v may have fewer heads than q (grouped-query attention, fa_forward_gqa)."""
    lib = load_library()
    hkv = _kv_heads(q, k, v)
    B, H, N, d = _shape(q)
    if k.dtype != q.dtype or k.device != q.device:
        raise ValueError("all tensors must share dtype and device")
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _shape(q, o)
    _check_lse(l, B, H, N, q.device)
    if hkv == H:
        _check(lib.fa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, N, d,
                              int(causal), scale, _DTYPE_CODE[q.dtype], _stream(q.device)))
    else:
        _check(lib.fa_forward_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, hkv, N, d,
                                  int(causal), scale, _DTYPE_CODE[q.dtype], _stream(q.device)))
    return o, l


def forward_blockmap(q, k, v, causal: bool = False, scale: float | None = None):
    """Instrumented forward: (O, LSE, tile_codes[B, H, nQ, nK] uint8)."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    br, bc = tile_config(0 if causal else 3, d, q.dtype)
    nq, nk = -(-N // br), -(-N // bc)
    o = torch.empty_like(q)
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    codes = torch.full((B, H, nq, nk), 255, dtype=torch.uint8, device=q.device)
    _check(lib.fa_forward_blockmap(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, N, d,
                                   int(causal), scale, _DTYPE_CODE[q.dtype], _ptr(codes),
                                   _stream(q.device)))
    return o, l, codes


def backward_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_backward_workspace_size(B, H, N, d))


def _check_lse(lse, B, H, N, device):
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous() \
            or lse.device != device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")


def backward(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
             workspace=None, out=None):
    """dQ, dK, dV of <dO, O> given the forward's O and LSE.

    `workspace` (float32, at least 2*B*H*N elements) and `out` = (dq, dk, dv) may be
    passed to avoid allocations."""
    lib = load_library()
    hkv = _kv_heads(q, k, v)
    B, H, N, d = _shape(q, o, do)
    if k.dtype != q.dtype or k.device != q.device:
        raise ValueError("all tensors must share dtype and device")
    scale = default_scale(d) if scale is None else float(scale)
    _check_lse(lse, B, H, N, q.device)
    ws = new_workspace(q, k) if workspace is None else workspace
    _check_workspace(ws, q.device)
    dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if out is None \
        else out
    _shape(q, dq)
    _shape(k, dk, dv)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv))
    rest = (N, d, int(causal), scale, _DTYPE_CODE[q.dtype], _ptr(ws),
            ws.numel() * ws.element_size(), _stream(q.device))
    if hkv == H:
        _check(lib.fa_backward(*args, B, H, *rest))
    else:
        _check(lib.fa_backward_gqa(*args, B, H, hkv, *rest))
    return dq, dk, dv


def backward_noalloc(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None,
                     out=None):
    """backward() through fa_backward_noalloc: the library's static scratch array
    replaces the workspace (B*H*N at most 2^20; multi-head attention only).  With
    `out` = (dq, dk, dv) nothing is allocated."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v, o, do)
    if k.dtype != q.dtype or k.device != q.device:
        raise ValueError("all tensors must share dtype and device")
    scale = default_scale(d) if scale is None else float(scale)
    _check_lse(lse, B, H, N, q.device)
    dq, dk, dv = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)) if out is None \
        else out
    _shape(q, dq, dk, dv)
    _check(lib.fa_backward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(causal), scale,
                                   _DTYPE_CODE[q.dtype], _stream(q.device)))
    return dq, dk, dv


def backward_blockmap(q, k, v, o, do, lse, causal: bool = False, scale: float | None = None):
    """Instrumented backward: (dq, dk, dv, dkdv_codes, dq_codes).

    dkdv_codes is [B, H, nK1, nQ1] (key tile major, tiles of tile_config(1, ...)),
    dq_codes is [B, H, nQ2, nK2] (tiles of tile_config(2, ...)), both uint8."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v, o, do)
    scale = default_scale(d) if scale is None else float(scale)
    _check_lse(lse, B, H, N, q.device)
    ws = new_workspace(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    br1, bc1 = tile_config(1, d, q.dtype)
    br2, bc2 = tile_config(2, d, q.dtype)
    c1 = torch.full((B, H, -(-N // bc1), -(-N // br1)), 255, dtype=torch.uint8, device=q.device)
    c2 = torch.full((B, H, -(-N // br2), -(-N // bc2)), 255, dtype=torch.uint8, device=q.device)
    _check(lib.fa_backward_blockmap(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                    _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(causal), scale,
                                    _DTYPE_CODE[q.dtype], _ptr(ws), ws.numel() * ws.element_size(),
                                    _ptr(c1), _ptr(c2), _stream(q.device)))
    return dq, dk, dv, c1, c2


def new_workspace(q: torch.Tensor, k: torch.Tensor | None = None) -> torch.Tensor:
    """Backward workspace for q [B, H, N, d] (and k [B, Hkv, N, d] when its heads are
    grouped)."""
    B, H, N, d = q.shape
    hkv = H if k is None else k.shape[1]
    nbytes = load_library().fa_backward_gqa_workspace_size(B, H, hkv, N, d)
    if nbytes == 0:
        raise ValueError("invalid backward shapes")
    return torch.empty(-(-nbytes // 4), dtype=torch.float32, device=q.device)


def backward_stage(stage: int, q, k, v, o, do, lse, dq, dk, dv, workspace, causal: bool = False,
                   scale: float | None = None):
    """Run one backward stage (BWD_PREPROCESS, BWD_DKDV or BWD_DQ) in place."""
    lib = load_library()
    B, H, N, d = _shape(q, k, v, o, do, dq, dk, dv)
    scale = default_scale(d) if scale is None else float(scale)
    _check_lse(lse, B, H, N, q.device)
    _check_workspace(workspace, q.device)
    _check(lib.fa_backward_stage(stage, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                 _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, int(causal), scale,
                                 _DTYPE_CODE[q.dtype], _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(q.device)))


# ------------------------------------------------------------------ split-K decode

def _decode_shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("expected q [B, H, Nq, d] and k, v [B, Hkv, Nk, d]")
    _shape(k, v)
    B, H, nq, d = q.shape
    if k.shape[0] != B or k.shape[3] != d or H % k.shape[1]:
        raise ValueError("q and k, v must agree in B and d, and Hkv must divide H")
    if q.dtype != k.dtype or q.device != k.device or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous GPU tensor of k's dtype and device")
    return B, H, k.shape[1], nq, k.shape[2], d


def decode_num_splits(B: int, H: int, hkv: int, nq: int, nk: int, d: int) -> int:
    """The slice count decode() uses by default."""
    n = int(load_library().fa_decode_num_splits(B, H, hkv, nq, nk, d))
    _check(min(n, 0))
    return n


def decode_workspace_size(B: int, H: int, hkv: int, nq: int, nk: int, d: int,
                          num_splits: int = 0) -> int:
    return int(load_library().fa_decode_workspace_size(B, H, hkv, nq, nk, d, num_splits))


def new_decode_workspace(q, k, num_splits: int = 0):
    B, H, nq, d = q.shape
    nbytes = decode_workspace_size(B, H, k.shape[1], nq, k.shape[2], d, num_splits)
    if nbytes == 0:
        raise ValueError("invalid decode shapes")
    return torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)


def decode(q, k, v, causal: bool = False, scale: float | None = None, num_splits: int = 0,
           workspace=None, out=None, lse=None):
    """Split-K decode: O [B, H, Nq, d] and LSE [B, H, Nq] of q against the cache k, v
    ([B, Hkv, Nk, d], Hkv dividing H: query head h reads key/value head h // (H // Hkv));
    the queries are the last Nq positions (causal: bottom-right)."""
    lib = load_library()
    B, H, hkv, nq, nk, d = _decode_shapes(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    ws = new_decode_workspace(q, k, num_splits) if workspace is None else workspace
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _shape(q, o)
    _check_lse(l, B, H, nq, q.device)
    _check_workspace(ws, q.device)
    _check(lib.fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, hkv, nq, nk, d,
                         int(causal), scale, _DTYPE_CODE[q.dtype], int(num_splits), _ptr(ws),
                         ws.numel() * ws.element_size(), _stream(q.device)))
    return o, l


def _check_workspace(ws, device) -> None:
    if ws.dtype != torch.float32 or ws.device != device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous float32 tensor on q's device")


def decode_stage(stage: int, q, k, v, o, lse, causal: bool, scale: float, num_splits: int,
                 workspace) -> None:
    """One kernel of decode(): DEC_SPLIT (writes the workspace) or DEC_COMBINE."""
    lib = load_library()
    B, H, hkv, nq, nk, d = _decode_shapes(q, k, v)
    _check_workspace(workspace, q.device)
    if o is not None:
        _shape(q, o)
    if lse is not None:
        _check_lse(lse, B, H, nq, q.device)
    _check(lib.fa_decode_stage(stage, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, hkv,
                               nq, nk, d, int(causal), float(scale), _DTYPE_CODE[q.dtype],
                               int(num_splits), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(q.device)))


# ------------------------------------------------------------------ FP8 input stage

def fp8_quantize_rows(x, signs=None, codes=None, scales=None):
    """Rows of x ([..., d], fp16/bf16, d = 64 or 128) rotated by diag(signs) H / sqrt(d)
    (no rotation when signs is None) and quantised to E4M3 with one fp32 scale per
    row: returns (codes uint8 [..., d], scales float32 [...]), x J ~= codes * scales.
    signs is a float32 tensor of d values, each +1 or -1, on x's device."""
    lib = load_library()
    if x.dim() < 1 or not x.is_cuda or not x.is_contiguous() or x.dtype not in _DTYPE_CODE:
        raise ValueError("x must be a contiguous fp16/bf16 GPU tensor")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if signs is not None and (signs.dtype != torch.float32 or tuple(signs.shape) != (d,)
                              or signs.device != x.device or not signs.is_contiguous()):
        raise ValueError("signs must be a contiguous float32 [d] tensor on x's device")
    c = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if codes is None else codes
    s = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if scales is None \
        else scales
    if c.dtype != torch.uint8 or c.shape != x.shape or c.device != x.device \
            or not c.is_contiguous():
        raise ValueError("codes must be a contiguous uint8 tensor of x's shape and device")
    if s.dtype != torch.float32 or s.shape != x.shape[:-1] or s.device != x.device \
            or not s.is_contiguous():
        raise ValueError("scales must be a contiguous float32 tensor of x's leading shape")
    _check(lib.fa_fp8_quantize_rows(_ptr(x), rows, d, _DTYPE_CODE[x.dtype], _ptr(signs), _ptr(c),
                                    _ptr(s), _stream(x.device)))
    return c, s


def forward_fp8(qc, qs, kc, ks, v, causal: bool = False, scale: float | None = None, out=None,
                lse=None):
    """O, LSE of the FP8 forward (fa_forward_fp8): qc, kc are E4M3 codes (uint8
    [B, H, N, d]) of Q J and K J with row scales qs, ks (float32 [B, H, N]), as
    fp8_quantize_rows returns them; v is fp16/bf16 [B, H, N, d]."""
    lib = load_library()
    B, H, N, d = _shape(v)
    for t, name in ((qc, "qc"), (kc, "kc")):
        if t.dtype != torch.uint8 or tuple(t.shape) != (B, H, N, d) or not t.is_contiguous() \
                or t.device != v.device:
            raise ValueError(f"{name} must be contiguous uint8 codes of v's shape and device")
    for t, name in ((qs, "qs"), (ks, "ks")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, N) or not t.is_contiguous() \
                or t.device != v.device:
            raise ValueError(f"{name} must be contiguous float32 [B, H, N] on v's device")
    if v.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("v must be fp16 or bf16")
    scale = default_scale(d) if scale is None else float(scale)
    o = torch.empty_like(v) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=v.device) if lse is None else lse
    _shape(v, o)
    _check_lse(l, B, H, N, v.device)
    _check(lib.fa_forward_fp8(_ptr(qc), _ptr(qs), _ptr(kc), _ptr(ks), _ptr(v), _ptr(o), _ptr(l), B,
                              H, N, d, int(causal), scale, _DTYPE_CODE[v.dtype],
                              _stream(v.device)))
    return o, l


def fp8_attention(q, k, v, signs, causal: bool = False, scale: float | None = None):
    """The FP8 path end to end: Q and K rotated by diag(signs) H / sqrt(d) and
    quantised to E4M3 per row (fp8_quantize_rows), then forward_fp8.  Returns
    (O, LSE, (qc, qs, kc, ks))."""
    qc, qs = fp8_quantize_rows(q, signs)
    kc, ks = fp8_quantize_rows(k, signs)
    o, l = forward_fp8(qc, qs, kc, ks, v, causal, scale)
    return o, l, (qc, qs, kc, ks)


__all__ = ["forward", "forward_blockmap", "backward", "backward_noalloc", "backward_blockmap",
           "backward_stage", "backward_workspace_size", "new_workspace", "tile_config",
           "decode", "decode_stage", "decode_num_splits", "decode_workspace_size",
           "new_decode_workspace", "fp8_quantize_rows", "forward_fp8", "fp8_attention",
           "default_scale", "load_library", "open_library", "FAError", "SYMBOLS", "LIB_PATH",
           "DEBUG_SYNC_LIB_PATH", "BWD_PREPROCESS", "BWD_DKDV", "BWD_DQ", "DEC_SPLIT",
           "DEC_COMBINE", "FA_F32", "FA_F16", "FA_BF16", "FA_OK", "FA_ERR_INVALID_ARG",
           "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP"]

"""MI355X-native SpargeAttn hot path: Python binding of libsparge (C ABI).

Every step of the path runs in the HIP kernels of ``libsparge.so``; this
module only marshals arguments (tensor pointers, sizes, strides, the current
HIP stream) and allocates outputs with PyTorch.  There is no CPU fallback: if
the library is not built, every call raises.

Entry points (names follow the C ABI in include/sparge.h):
  predict_mask(q, k, tau, theta, causal)        -> Mask (mg, row_cnt, row_idx, s_q, s_k)
  attn(q, k, v, mask_or_mg, lam, causal, ...)   -> (o, counts, pv_dbg or None)
  quant_qk_int8(q, k)                           -> (q8, k8, q_scale, k_scale)
  hilbert_index(T, H, W)                        -> (perm, inv) as numpy int32 (host)
  hilbert_permute(x, perm, inverse)             -> y
  grid_order(T, H, W, order)                    -> (perm, inv): Hilbert, raster or time-fastest
  l1_sums(o, ref) / l1_error(o, ref)            -> relative L1 of O' against O
  sparge_attention(q, k, v, tau, theta, lam, causal, ...) -> the whole path
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsparge.so")

SPARGE_OK = 0
SPARGE_EINVAL = -1
SPARGE_EUNSUPPORTED = -2
SPARGE_EWORKSPACE = -3
SPARGE_EHIP = -4
F16, BF16, I8, F32 = 0, 1, 2, 3
PATH_AUTO, PATH_TWO_PASS, PATH_FUSED = 0, 1, 2
ORDER_HILBERT, ORDER_ROWMAJOR, ORDER_TIMEMAJOR = 0, 1, 2
BQ, BK = 128, 64
COUNTER_NAMES = ("live_tiles", "qk_exec", "qk_skip", "pv_exec", "pv_skip", "pv_void",
                 "empty_rows", "rows")


class SpargeError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


class SpargeTensor(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d", ctypes.c_int64), ("sb", ctypes.c_int64), ("sh", ctypes.c_int64),
                ("sn", ctypes.c_int64)]


_vp = ctypes.c_void_p
_TP = ctypes.POINTER(SpargeTensor)
_SIGNATURES = {
    "sparge_version": (ctypes.c_int, []),
    "sparge_last_error": (ctypes.c_char_p, []),
    "sparge_rows_per_wave": (ctypes.c_int, []),
    "sparge_workspace_size": (ctypes.c_size_t, [_TP, _TP]),
    "sparge_attn_path": (ctypes.c_int, [ctypes.c_int]),
    "sparge_hilbert_index": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "sparge_hilbert_permute": (ctypes.c_int, [_vp, _TP, _vp, _TP, ctypes.c_int, _vp, ctypes.c_int, _vp]),
    "sparge_quant_qk_int8": (ctypes.c_int, [_vp, _TP, _vp, _TP, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                            ctypes.c_size_t, _vp]),
    "sparge_predict_mask": (ctypes.c_int, [_vp, _TP, _vp, _TP, ctypes.c_int, ctypes.c_double,
                                           ctypes.c_double, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                           ctypes.c_size_t, _vp]),
    "sparge_attn": (ctypes.c_int, [_vp, _TP, _vp, _TP, _vp, _TP, _vp, _TP, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, ctypes.c_int,
                                   _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "sparge_attn_fp8pv": (ctypes.c_int, [_vp, _TP, _vp, _TP, _vp, _TP, _vp, _TP, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, ctypes.c_int,
                                         _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "sparge_attn_noalloc": (ctypes.c_int, [_vp, _TP, _vp, _TP, _vp, _TP, _vp, _TP, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, ctypes.c_int,
                                           _vp, _vp, _vp]),
    "sparge_grid_order": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "sparge_l1_workspace_size": (ctypes.c_size_t, []),
    "sparge_l1_sums": (ctypes.c_int, [_vp, _TP, ctypes.c_int, _vp, _TP, ctypes.c_int, _vp, _vp,
                                      ctypes.c_size_t, _vp]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libsparge.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m free_block_sparse_mask_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, rc: int) -> None:
    if rc != SPARGE_OK:
        raise SpargeError(fn, rc, lib().sparge_last_error().decode())


def rows_per_wave() -> int:
    return lib().sparge_rows_per_wave()


def attn_path(path: Optional[int] = None) -> int:
    """The stage-2 path of later calls, process-wide (sparge_attn_path):
    PATH_AUTO (a pilot on the device chooses per call), PATH_TWO_PASS or
    PATH_FUSED.  With ``path`` None, only returns the current setting;
    otherwise sets it and returns the previous one."""
    rc = lib().sparge_attn_path(-1 if path is None else int(path))
    if rc < 0:
        _check("sparge_attn_path", rc)
    return rc


def desc(x) -> SpargeTensor:
    """Descriptor of a 4-D [B, heads, N, d] tensor whose last axis is contiguous."""
    if x.dim() != 4:
        raise ValueError(f"expected a 4-D [B, heads, N, d] tensor, got shape {tuple(x.shape)}")
    if x.shape[3] > 1 and x.stride(3) != 1:
        raise ValueError("the last (d) axis must be contiguous")
    B, H, N, d = x.shape
    sb, sh, sn = x.stride(0), x.stride(1), x.stride(2)
    return SpargeTensor(B, H, N, d, sb, sh, sn)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.int8:
        return I8
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


_workspaces = {}


def workspace(q, k):
    """A cached device workspace large enough for (q, k) on q's device.  Every
    call rewrites it, so calls on one stream may share it; calls that can run
    at the same time (other streams) need workspaces of their own (``ws=``)."""
    import torch
    need = lib().sparge_workspace_size(ctypes.byref(desc(q)), ctypes.byref(desc(k)))
    dev = q.device
    ws = _workspaces.get(dev)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _workspaces[dev] = ws
    return ws


def num_blocks(N: int, b: int) -> int:
    return (N + b - 1) // b


@dataclasses.dataclass
class Mask:
    mg: "object"          # uint8 [B, H, Tm, Tn]
    row_cnt: "object"     # int32 [B, H, Tm]
    row_idx: "object"     # int16 storage of uint16 [B, H, Tm, Tn]
    s_q: "object"         # float64 [B, H, Tm]
    s_k: "object"         # float64 [B, H_kv, Tn]


def predict_mask(q, k, tau: float, theta: float, causal: bool, ws=None) -> Mask:
    """Stage 1 (sparge_predict_mask): M_g and its compacted row lists."""
    import torch
    B, H, N, _ = q.shape
    Hkv = k.shape[1]
    Tm, Tn = num_blocks(N, BQ), num_blocks(N, BK)
    dev = q.device
    mg = torch.empty((B, H, Tm, Tn), dtype=torch.uint8, device=dev)
    cnt = torch.empty((B, H, Tm), dtype=torch.int32, device=dev)
    idx = torch.empty((B, H, Tm, Tn), dtype=torch.int16, device=dev)
    s_q = torch.empty((B, H, Tm), dtype=torch.float64, device=dev)
    s_k = torch.empty((B, Hkv, Tn), dtype=torch.float64, device=dev)
    ws = workspace(q, k) if ws is None else ws
    rc = lib().sparge_predict_mask(_ptr(q), ctypes.byref(desc(q)), _ptr(k), ctypes.byref(desc(k)),
                                   _dtype_code(q), float(tau), float(theta), int(bool(causal)),
                                   _ptr(mg), _ptr(cnt), _ptr(idx), _ptr(s_q), _ptr(s_k), _ptr(ws),
                                   ws.numel(), _stream(dev))
    _check("sparge_predict_mask", rc)
    return Mask(mg, cnt, idx, s_q, s_k)


def attn(q, k, v, mask, lam: float, causal: bool, q_scale=None, k_scale=None, counts=None,
         dbg: bool = False, out=None, ws=None, out_f32: bool = False, fp8_pv: bool = False,
         noalloc: bool = False):
    """Stage 2 (sparge_attn, sparge_attn_fp8pv with ``fp8_pv``, or
    sparge_attn_noalloc with ``noalloc``: no workspace, the library's static
    scratch instead).  ``mask`` is a :class:`Mask` (its row lists are used)
    or a uint8 M_g tensor [B, H, Tm, Tn] (lists are built on the device).
    ``out_f32`` stores O in float32 (before its rounding to V's type).
    Returns (o, counts int64[8] on the device, pv_dbg or None)."""
    import torch
    B, H, N, d = q.shape
    dev = q.device
    Tm, Tn = num_blocks(N, BQ), num_blocks(N, BK)
    if isinstance(mask, Mask):
        mg, cnt, idx = mask.mg, mask.row_cnt, mask.row_idx
    else:
        mg, cnt, idx = mask, None, None
    if out is None:
        o = torch.empty((B, H, N, d), dtype=torch.float32 if out_f32 else v.dtype, device=dev)
    else:
        o = out
    counts = torch.empty(8, dtype=torch.int64, device=dev) if counts is None else counts
    pv_dbg = torch.zeros((B, H, Tm, Tn, BQ // 32), dtype=torch.uint8, device=dev) if dbg else None
    if noalloc:
        if fp8_pv:
            raise ValueError("the entry point without a workspace has no fp8 P~V form")
        rc = lib().sparge_attn_noalloc(_ptr(q), ctypes.byref(desc(q)), _ptr(k), ctypes.byref(desc(k)),
                                       _ptr(v), ctypes.byref(desc(v)), _ptr(o), ctypes.byref(desc(o)),
                                       _dtype_code(q), _dtype_code(v), _dtype_code(o), _ptr(q_scale),
                                       _ptr(k_scale), _ptr(mg), _ptr(cnt), _ptr(idx), float(lam),
                                       int(bool(causal)), _ptr(counts), _ptr(pv_dbg), _stream(dev))
        _check("sparge_attn_noalloc", rc)
        return o, counts, pv_dbg
    ws = workspace(q, k) if ws is None else ws
    fn = lib().sparge_attn_fp8pv if fp8_pv else lib().sparge_attn
    rc = fn(_ptr(q), ctypes.byref(desc(q)), _ptr(k), ctypes.byref(desc(k)),
                           _ptr(v), ctypes.byref(desc(v)), _ptr(o), ctypes.byref(desc(o)),
                           _dtype_code(q), _dtype_code(v), _dtype_code(o), _ptr(q_scale),
                           _ptr(k_scale), _ptr(mg),
                           _ptr(cnt), _ptr(idx), float(lam), int(bool(causal)), _ptr(counts),
                           _ptr(pv_dbg), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev))
    _check("sparge_attn_fp8pv" if fp8_pv else "sparge_attn", rc)
    return o, counts, pv_dbg


def quant_qk_int8(q, k, ws=None):
    """int8 per-block codes of Q and of K minus its token mean (sparge_quant_qk_int8)."""
    import torch
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    dev = q.device
    q8 = torch.empty((B, H, N, d), dtype=torch.int8, device=dev)
    k8 = torch.empty((B, Hkv, N, d), dtype=torch.int8, device=dev)
    qs = torch.empty((B, H, num_blocks(N, BQ)), dtype=torch.float32, device=dev)
    ks = torch.empty((B, Hkv, num_blocks(N, BK)), dtype=torch.float32, device=dev)
    ws = workspace(q, k) if ws is None else ws
    rc = lib().sparge_quant_qk_int8(_ptr(q), ctypes.byref(desc(q)), _ptr(k), ctypes.byref(desc(k)),
                                    _dtype_code(q), _ptr(q8), _ptr(k8), _ptr(qs), _ptr(ks), _ptr(ws),
                                    ws.numel(), _stream(dev))
    _check("sparge_quant_qk_int8", rc)
    return q8, k8, qs, ks


def hilbert_index(T: int, H: int, W: int):
    """Host-side 3D Hilbert order: (perm, inv) int32 numpy arrays of T*H*W tokens."""
    n = T * H * W
    perm = np.empty(n, dtype=np.int32)
    inv = np.empty(n, dtype=np.int32)
    rc = lib().sparge_hilbert_index(T, H, W, perm.ctypes.data, inv.ctypes.data)
    _check("sparge_hilbert_index", rc)
    return perm, inv


def hilbert_permute(x, perm, inverse: bool = False, out=None):
    """Token gather (inverse=False) or scatter (inverse=True) along N on the device."""
    import torch
    y = torch.empty_like(x, memory_format=torch.contiguous_format) if out is None else out
    rc = lib().sparge_hilbert_permute(_ptr(x), ctypes.byref(desc(x)), _ptr(y), ctypes.byref(desc(y)),
                                      _dtype_code(x), _ptr(perm), int(bool(inverse)), _stream(x.device))
    _check("sparge_hilbert_permute", rc)
    return y


def grid_order(T: int, H: int, W: int, order: int):
    """Host-side token order of a T x H x W grid (sparge_grid_order):
    ORDER_HILBERT, ORDER_ROWMAJOR or ORDER_TIMEMAJOR; (perm, inv) int32 numpy."""
    n = T * H * W
    perm = np.empty(n, dtype=np.int32)
    inv = np.empty(n, dtype=np.int32)
    rc = lib().sparge_grid_order(T, H, W, order, perm.ctypes.data, inv.ctypes.data)
    _check("sparge_grid_order", rc)
    return perm, inv


def l1_sums(o, ref, out=None):
    """Device float64 [sum|o - ref|, sum|ref|] (sparge_l1_sums), same bits on every call."""
    import torch
    dev = o.device
    out = torch.empty(2, dtype=torch.float64, device=dev) if out is None else out
    need = lib().sparge_l1_workspace_size()
    ws = _l1_ws.get(dev)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        _l1_ws[dev] = ws
    rc = lib().sparge_l1_sums(_ptr(o), ctypes.byref(desc(o)), _dtype_code(o), _ptr(ref),
                              ctypes.byref(desc(ref)), _dtype_code(ref), _ptr(out), _ptr(ws),
                              ws.numel(), _stream(dev))
    _check("sparge_l1_sums", rc)
    return out


_l1_ws = {}


def l1_error(o, ref) -> float:
    """Relative L1 error sum|o - ref| / sum|ref| (0 when ref is all zero)."""
    s = l1_sums(o, ref).cpu().tolist()
    return s[0] / s[1] if s[1] > 0 else 0.0


def counts_dict(counts) -> dict:
    vals = counts.cpu().tolist() if hasattr(counts, "cpu") else list(counts)
    return dict(zip(COUNTER_NAMES, (int(v) for v in vals)))


def sparge_attention(q, k, v, tau: float, theta: float, lam: float, causal: bool,
                     int8: bool = False, perm=None):
    """The whole hot path: [Hilbert gather] -> [int8 quantisation] -> predict
    M_g -> sparse attention -> [Hilbert scatter].  ``perm`` is a device int32
    token order (from :func:`hilbert_index`), applied to Q, K, V and undone on O.
    With ``int8``, V must be float16 or bfloat16 and sets the P~V type."""
    if perm is not None:
        q, k, v = (hilbert_permute(x, perm) for x in (q, k, v))
    mask = predict_mask(q, k, tau, theta, causal)
    if int8:
        q8, k8, qs, ks = quant_qk_int8(q, k)
        o, counts, _ = attn(q8, k8, v, mask, lam, causal, q_scale=qs, k_scale=ks)
    else:
        o, counts, _ = attn(q, k, v, mask, lam, causal)
    if perm is not None:
        o = hilbert_permute(o, perm, inverse=True)
    return o, mask, counts

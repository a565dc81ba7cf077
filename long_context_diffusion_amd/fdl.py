"""Python binding of the C ABI in include/fdl.h (libfdl.so, gfx950).

Argument marshalling only: every step of the sparse attention path runs in the
library's HIP kernels.  PyTorch provides device memory and the current stream.
Functions take torch tensors on the GPU, pass their data pointers, sizes and
element strides to the library, and return output tensors (allocated here when
the caller passes none).  A missing library, or a status other than FDL_OK,
raises FdlError: there is no fallback path.

Entry points (same names as the C functions without the fdl_ prefix):
  pcgi_select, dense_attention, sink_identify, block_means, block_score_topc, sparse_attention.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfdl.so")

FDL_F32, FDL_BF16 = 0, 1
STATUS = {0: "FDL_OK", 1: "FDL_ERR_NULL", 2: "FDL_ERR_SHAPE", 3: "FDL_ERR_DTYPE", 4: "FDL_ERR_ALIGN",
          5: "FDL_ERR_WORKSPACE", 6: "FDL_ERR_HIP", 7: "FDL_ERR_UNSUPPORTED"}
EXPORTS = (
    "fdl_status_string", "fdl_focus_count",
    "fdl_pcgi_select",
    "fdl_dense_attention_workspace_bytes", "fdl_dense_attention",
    "fdl_sink_identify_workspace_bytes", "fdl_sink_identify",
    "fdl_block_means", "fdl_block_score_topc_workspace_bytes", "fdl_block_score_topc",
    "fdl_sparse_attention_workspace_bytes", "fdl_sparse_attention",
    "fdl_kv_refresh", "fdl_block_means_refresh",
    "fdl_block_score_topc_noalloc_max_bytes", "fdl_block_score_topc_noalloc",
    "fdl_confidence_unmask_workspace_bytes", "fdl_confidence_unmask",
    "fdl_dcu_select_workspace_bytes", "fdl_dcu_select",
    "fdl_block_score_topc_ex", "fdl_sparse_attention_ex_workspace_bytes", "fdl_sparse_attention_ex",
    "fdl_calibrate_read", "fdl_calibrate_mfma", "fdl_kv_refresh_means",
)
FDL_SCORE_PER_HEAD, FDL_SCORE_MAX = 1, 2


class FdlError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_text(status)})")


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("r", ctypes.c_int64)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_D = ctypes.c_double

_SIGS = {
    "fdl_status_string": (ctypes.c_char_p, [_I]),
    "fdl_focus_count": (_I, [_I, _D]),
    "fdl_pcgi_select": (_I, [_P, _P, _I, _I, _I, _D, _I, _P, _P, _I, _P, _P, _I, _P]),
    "fdl_dense_attention_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "fdl_dense_attention": (_I, [_I, _I, _I, _I, _I, _I, _P, Strides, _P, _P, _I, _P, Strides, _P, Strides, _P, Strides,
                                 _F, _P, Strides, _P, _P, _SZ, _P]),
    "fdl_sink_identify_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "fdl_sink_identify": (_I, [_I, _I, _I, _I, _I, _I, _P, Strides, _P, _P, _I, _P, Strides, _F, _P, _I,
                               _P, _P, _P, _SZ, _P]),
    "fdl_block_means": (_I, [_I, _I, _I, _I, _I, _I, _P, Strides, _I, _P, _P]),
    "fdl_block_score_topc_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "fdl_block_score_topc": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, Strides, _P, _P, _I, _P, Strides, _F,
                                  _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "fdl_sparse_attention_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "fdl_kv_refresh": (_I, [_I, _I, _I, _I, _I, _P, _P, _I, _P, Strides, _P, Strides, _P, Strides, _P, Strides,
                            _P, Strides, _P]),
    "fdl_block_means_refresh": (_I, [_I, _I, _I, _I, _I, _I, _P, Strides, _I, _P, _P, _I, _P, _P]),
    "fdl_block_score_topc_noalloc_max_bytes": (_SZ, []),
    "fdl_confidence_unmask_workspace_bytes": (_SZ, [_I, _I, _I]),
    "fdl_confidence_unmask": (_I, [_I, _I, _I, _I, _P, Strides, _P, _P, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "fdl_dcu_select_workspace_bytes": (_SZ, [_I, _I, _I]),
    "fdl_block_score_topc_ex": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, Strides, _P, _P, _I, _P, Strides, _F,
                                     _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "fdl_sparse_attention_ex_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "fdl_sparse_attention_ex": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, Strides, _P, _P, _I, _P, Strides, _P,
                                     Strides, _P, Strides, _P, _I, _P, _I, _I, _I, _F, _P, Strides, _P, _P, _SZ,
                                     _P]),
    "fdl_dcu_select": (_I, [_I, _I, _I, _I, _I, _P, Strides, _P, Strides, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                            _SZ, _P]),
    "fdl_calibrate_read": (_I, [_P, _SZ, _P, _I, _P]),
    "fdl_kv_refresh_means": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, Strides, _P, Strides, _P, Strides,
                                  _P, Strides, _P, Strides, _P, _P]),
    "fdl_calibrate_mfma": (_I, [_I, _I, _F, _F, _P, _P]),
    "fdl_block_score_topc_noalloc": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, Strides, _P, _P, _I, _P, Strides, _F,
                                          _I, _I, _P, _P, _P, _P]),
    "fdl_sparse_attention": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, Strides, _P, _P, _I, _P, Strides, _P,
                                  Strides, _P, Strides, _P, _I, _P, _I, _I, _F, _P, Strides, _P, _P, _SZ, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfdl.so with argument types set; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FdlError(-1, f"{LIB_PATH} is missing; build it with long_context_diffusion_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _status_text(status: int) -> str:
    try:
        return lib().fdl_status_string(status).decode()
    except Exception:  # library not loadable
        return "?"


def _check(status: int, what: str):
    if status != 0:
        raise FdlError(status, what)


# ------------------------------------------------------------------ marshalling helpers

def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FDL_BF16
    if t.dtype == torch.float32:
        return FDL_F32
    raise FdlError(3, f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides4(t: torch.Tensor) -> Strides:
    """Element strides of a [B, H, rows, d] tensor whose last axis is contiguous."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise FdlError(2, "expected a [B, H, rows, d] tensor with a contiguous last axis")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _vt(vt, v):
    """Pointer and (b, h, d) strides of an optional [B, Hkv, d, L] V^T with contiguous keys."""
    if vt is None:
        return None, Strides(0, 0, 0)
    B, H, L, d = v.shape
    if tuple(vt.shape) != (B, H, d, L) or vt.dtype != v.dtype or vt.device != v.device:
        raise FdlError(2, f"vt must be a [B, Hkv, d, L] tensor like v, got {tuple(vt.shape)}")
    return _ptr(vt), _strides4(vt)


def transpose_v(v: torch.Tensor) -> torch.Tensor:
    """A [B, H, d, L] copy of v [B, H, L, d] with the keys contiguous (the vt argument).

    The rows are padded to a multiple of 8 keys, so every stride is 16-byte aligned."""
    B, H, L, d = v.shape
    Lp = (L + 7) // 8 * 8
    buf = torch.empty((B, H, d, Lp), dtype=v.dtype, device=v.device)
    buf[..., :L].copy_(v.transpose(2, 3))
    return buf[..., :L]


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Workspace:
    """A reusable device byte buffer, grown on demand (allocation outside the library)."""

    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return ctypes.c_void_p(self.buf.data_ptr()), self.buf.numel()


_default_ws = {}


def _ws(workspace, device):
    if workspace is None:
        key = str(device)
        if key not in _default_ws:
            _default_ws[key] = Workspace(device)
        workspace = _default_ws[key]
    return workspace


def focus_count(n_t: int, rho: float) -> int:
    return int(lib().fdl_focus_count(int(n_t), float(rho)))


# ------------------------------------------------------------------ entry points

def pcgi_select(conf, mask, n_t: int, rho: float, w: int, *, k_cap=None, nq_max=None, out=None,
                stream=None):
    """I_focus and I_active (fdl_pcgi_select).  conf [B, L] fp32, mask [B, L] uint8.

    Returns (focus_idx [B, k_cap], n_focus [B], active_idx [B, nq_max], n_active [B]), int32.
    """
    B, L = conf.shape
    k = focus_count(n_t, rho)
    k_cap = max(k, 1) if k_cap is None else k_cap
    nq_max = max(min(k * w, L), 1) if nq_max is None else nq_max
    dev = conf.device
    if out is None:
        out = (torch.empty((B, k_cap), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev),
               torch.empty((B, nq_max), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    focus_idx, n_focus, active_idx, n_active = out
    st = lib().fdl_pcgi_select(_ptr(conf), _ptr(mask), B, L, int(n_t), float(rho), int(w),
                               _ptr(focus_idx), _ptr(n_focus), k_cap, _ptr(active_idx), _ptr(n_active),
                               nq_max, _stream(stream))
    _check(st, "fdl_pcgi_select")
    return focus_idx, n_focus, active_idx, n_active


def _rows(q, q_idx, n_q, nq_max):
    if nq_max is None:
        nq_max = q_idx.shape[1] if q_idx is not None else q.shape[2]
    return _ptr(q_idx), _ptr(n_q), int(nq_max)


def dense_attention_workspace_bytes(dtype_code, B, Hq, Hkv, L, d, nq_max) -> int:
    return int(lib().fdl_dense_attention_workspace_bytes(dtype_code, B, Hq, Hkv, L, d, nq_max))


def dense_attention(q, k, v, *, vt=None, q_idx=None, n_q=None, nq_max=None, scale: float = 0.0, out=None,
                    lse=None, want_lse=True, workspace=None, stream=None):
    """Full attention of the selected query rows over all keys (fdl_dense_attention).

    q [B, Hq, rows, d]; k, v [B, Hkv, L, d]; vt None or transpose_v(v).
    Returns (o [B, Hq, nq_max, d], lse [B, Hq, nq_max] or None).
    """
    B, Hq, _, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    qi, nqp, nq_max = _rows(q, q_idx, n_q, nq_max)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, Hq, nq_max, d), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, nq_max), dtype=torch.float32, device=q.device)
    ws, ws_n = _ws(workspace, q.device).get(dense_attention_workspace_bytes(dt, B, Hq, Hkv, L, d, nq_max))
    st = lib().fdl_dense_attention(dt, B, Hq, Hkv, L, d, _ptr(q), _strides4(q), qi, nqp, nq_max,
                                   _ptr(k), _strides4(k), _ptr(v), _strides4(v), *_vt(vt, v), float(scale),
                                   _ptr(out), _strides4(out), _ptr(lse), ws, ws_n, _stream(stream))
    _check(st, "fdl_dense_attention")
    return out, lse


def sink_identify(q, k, lse, n_sinks: int, *, q_idx=None, n_q=None, nq_max=None, scale: float = 0.0,
                  out=None, scores=None, want_scores=False, workspace=None, stream=None):
    """Attention-sink positions at layer l_dense (fdl_sink_identify).

    Returns (sink_idx [B, n_sinks] int32, scores [B, L] fp32 or None).
    """
    B, Hq, _, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    qi, nqp, nq_max = _rows(q, q_idx, n_q, nq_max)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, max(n_sinks, 1)), dtype=torch.int32, device=q.device)
    if scores is None and want_scores:
        scores = torch.empty((B, L), dtype=torch.float32, device=q.device)
    nbytes = int(lib().fdl_sink_identify_workspace_bytes(dt, B, Hq, Hkv, L, d, nq_max))
    ws, ws_n = _ws(workspace, q.device).get(nbytes)
    st = lib().fdl_sink_identify(dt, B, Hq, Hkv, L, d, _ptr(q), _strides4(q), qi, nqp, nq_max,
                                 _ptr(k), _strides4(k), float(scale), _ptr(lse), int(n_sinks),
                                 _ptr(out), _ptr(scores), ws, ws_n, _stream(stream))
    _check(st, "fdl_sink_identify")
    return out[:, :n_sinks], scores


def block_means(k, P: int, bs: int, *, out=None, stream=None):
    """Mean key of every prompt block (fdl_block_means): [B, Hkv, nb, d] fp32."""
    B, Hkv, L, d = k.shape
    nb = -(-P // bs)
    if out is None:
        out = torch.empty((B, Hkv, nb, d), dtype=torch.float32, device=k.device)
    if tuple(out.shape) != (B, Hkv, nb, d) or out.dtype != torch.float32 or not out.is_contiguous():
        raise FdlError(2, "block means: expected a contiguous [B, Hkv, nb, d] fp32 output")
    st = lib().fdl_block_means(_dtype_code(k), B, Hkv, L, P, d, _ptr(k), _strides4(k), int(bs), _ptr(out),
                               _stream(stream))
    _check(st, "fdl_block_means")
    return out


def kv_refresh(rows, k_new, v_new, k, v, *, n_rows=None, vt=None, stream=None):
    """Approximate KV cache refresh (fdl_kv_refresh): rows [B, n_max] int32 (-1 skipped),
    k_new, v_new [B, Hkv, n_max, d] into the caches k, v [B, Hkv, L, d] (and vt, when given)."""
    B, Hkv, L, d = k.shape
    n_max = rows.shape[1]
    if rows.dtype != torch.int32 or not rows.is_contiguous():
        raise FdlError(2, "rows must be a contiguous int32 [B, n_max] tensor")
    if tuple(k_new.shape) != (B, Hkv, n_max, d) or tuple(v_new.shape) != (B, Hkv, n_max, d):
        raise FdlError(2, "k_new, v_new must be [B, Hkv, n_max, d]")
    vtp, vts = _vt(vt, v)
    st = lib().fdl_kv_refresh(_dtype_code(k), B, Hkv, L, d, _ptr(rows), _ptr(n_rows), n_max, _ptr(k_new),
                              _strides4(k_new), _ptr(v_new), _strides4(v_new), _ptr(k), _strides4(k), _ptr(v),
                              _strides4(v), vtp, vts, _stream(stream))
    _check(st, "fdl_kv_refresh")


def kv_refresh_means(rows, k_new, v_new, k, v, P: int, bs: int, kbar, *, n_rows=None, vt=None, stream=None):
    """kv_refresh and block_means_refresh of the same rows in one launch (fdl_kv_refresh_means)."""
    B, Hkv, L, d = k.shape
    n_max = rows.shape[1]
    nb = -(-P // bs)
    if rows.dtype != torch.int32 or not rows.is_contiguous():
        raise FdlError(2, "rows must be a contiguous int32 [B, n_max] tensor")
    if tuple(k_new.shape) != (B, Hkv, n_max, d) or tuple(v_new.shape) != (B, Hkv, n_max, d):
        raise FdlError(2, "k_new, v_new must be [B, Hkv, n_max, d]")
    if tuple(kbar.shape) != (B, Hkv, nb, d) or kbar.dtype != torch.float32 or not kbar.is_contiguous():
        raise FdlError(2, "block means: expected a contiguous [B, Hkv, nb, d] fp32 kbar")
    vtp, vts = _vt(vt, v)
    st = lib().fdl_kv_refresh_means(_dtype_code(k), B, Hkv, L, P, d, int(bs), _ptr(rows), _ptr(n_rows), n_max,
                                    _ptr(k_new), _strides4(k_new), _ptr(v_new), _strides4(v_new), _ptr(k),
                                    _strides4(k), _ptr(v), _strides4(v), vtp, vts, _ptr(kbar), _stream(stream))
    _check(st, "fdl_kv_refresh_means")
    return kbar


def block_means_refresh(k, P: int, bs: int, rows, kbar, *, n_rows=None, stream=None):
    """The block means a refresh touched (fdl_block_means_refresh), recomputed in kbar."""
    B, Hkv, L, d = k.shape
    nb = -(-P // bs)
    if tuple(kbar.shape) != (B, Hkv, nb, d) or kbar.dtype != torch.float32 or not kbar.is_contiguous():
        raise FdlError(2, "block means: expected a contiguous [B, Hkv, nb, d] fp32 kbar")
    if rows.dtype != torch.int32 or not rows.is_contiguous():
        raise FdlError(2, "rows must be a contiguous int32 [B, n_max] tensor")
    st = lib().fdl_block_means_refresh(_dtype_code(k), B, Hkv, L, P, d, _ptr(k), _strides4(k), int(bs),
                                       _ptr(rows), _ptr(n_rows), rows.shape[1], _ptr(kbar), _stream(stream))
    _check(st, "fdl_block_means_refresh")
    return kbar


def block_score_topc(q, k, P: int, bs: int, C: int, *, q_idx=None, n_q=None, nq_max=None,
                     scale: float = 0.0, out=None, want_R=False, want_kbar=False, kbar=None, L=None,
                     per_head=False, aggregator="sum", workspace=None, stream=None):
    """Top-C prompt blocks by relevance to the active queries (fdl_block_score_topc, or
    fdl_block_score_topc_ex for per_head / aggregator "max").

    k None: kbar must hold the block means (block_means) and L the sequence length.
    Returns (block_idx [B, C] int32 ([B, Hkv, C] per head), R [B, nb] ([B, Hkv, nb]) fp64 or
    None, kbar [B, Hkv, nb, d] fp32 or None).
    """
    B, Hq, _, d = q.shape
    if k is not None:
        Hkv, L = k.shape[1], k.shape[2]
    else:
        if kbar is None or L is None:
            raise FdlError(1, "block_score_topc without keys needs kbar and L")
        Hkv = kbar.shape[1]
    if aggregator not in ("sum", "max"):
        raise FdlError(2, f"unknown relevance aggregator {aggregator!r}")
    mode = (FDL_SCORE_PER_HEAD if per_head else 0) | (FDL_SCORE_MAX if aggregator == "max" else 0)
    qi, nqp, nq_max = _rows(q, q_idx, n_q, nq_max)
    dt = _dtype_code(q)
    nb = -(-P // bs)
    lead = (B, Hkv) if per_head else (B,)
    if out is None:
        out = torch.empty(lead + (max(C, 1),), dtype=torch.int32, device=q.device)
    R = torch.empty(lead + (nb,), dtype=torch.float64, device=q.device) if want_R else None
    if kbar is None and want_kbar:
        kbar = torch.empty((B, Hkv, nb, d), dtype=torch.float32, device=q.device)
    nbytes = int(lib().fdl_block_score_topc_workspace_bytes(dt, B, Hq, Hkv, P, d, bs, nq_max))
    ws, ws_n = _ws(workspace, q.device).get(nbytes)
    ks = _strides4(k) if k is not None else Strides(0, 0, d)
    st = lib().fdl_block_score_topc_ex(dt, B, Hq, Hkv, L, P, d, _ptr(q), _strides4(q), qi, nqp, nq_max,
                                       _ptr(k), ks, float(scale), int(bs), int(C), mode, _ptr(out),
                                       _ptr(R), _ptr(kbar), ws, ws_n, _stream(stream))
    _check(st, "fdl_block_score_topc_ex")
    return out[..., :C], R, kbar


def sparse_attention(q, k, v, P: int, sink_idx, block_idx, bs: int, *, vt=None, q_idx=None, n_q=None,
                     nq_max=None, scale: float = 0.0, out=None, lse=None, want_lse=False,
                     workspace=None, stream=None):
    """Attention of the active queries over I_p only (fdl_sparse_attention_ex).

    sink_idx [B, n_sinks] and block_idx [B, C] int32 or None: each read as the set of its
    valid entries (any order, repeats count once, -1 and out-of-range entries ignored); a
    [B, Hkv, C] block_idx gives every KV head its own blocks.  vt None or transpose_v(v).
    Returns (o [B, Hq, nq_max, d], lse or None).
    """
    B, Hq, _, d = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    qi, nqp, nq_max = _rows(q, q_idx, n_q, nq_max)
    dt = _dtype_code(q)
    n_sinks = 0 if sink_idx is None else sink_idx.shape[1]
    per_head = block_idx is not None and block_idx.dim() == 3
    if per_head and tuple(block_idx.shape[:2]) != (B, Hkv):
        raise FdlError(2, "per-head block_idx must be [B, Hkv, C]")
    C = 0 if block_idx is None else block_idx.shape[-1]
    if sink_idx is not None and sink_idx.stride(1) != 1 or (block_idx is not None and block_idx.stride(-1) != 1):
        raise FdlError(2, "index tensors must be contiguous along their last axis")
    if sink_idx is not None and n_sinks and sink_idx.stride(0) != n_sinks:
        sink_idx = sink_idx.contiguous()
    if block_idx is not None and C and not block_idx.is_contiguous():
        block_idx = block_idx.contiguous()
    if out is None:
        out = torch.empty((B, Hq, nq_max, d), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, nq_max), dtype=torch.float32, device=q.device)
    nbytes = int(lib().fdl_sparse_attention_ex_workspace_bytes(dt, B, Hq, Hkv, L, P, d, nq_max, n_sinks, C, bs,
                                                                int(per_head)))
    ws, ws_n = _ws(workspace, q.device).get(nbytes)
    st = lib().fdl_sparse_attention_ex(dt, B, Hq, Hkv, L, P, d, _ptr(q), _strides4(q), qi, nqp, nq_max,
                                       _ptr(k), _strides4(k), _ptr(v), _strides4(v), *_vt(vt, v), _ptr(sink_idx),
                                       n_sinks, _ptr(block_idx), C, int(per_head), int(bs), float(scale), _ptr(out),
                                       _strides4(out), _ptr(lse), ws, ws_n, _stream(stream))
    _check(st, "fdl_sparse_attention_ex")
    return out, lse


def confidence_unmask(logits, pos, mask, conf, n_t: int, *, n_rows=None, tokens=None, unmasked=None,
                      want_unmasked=True, workspace=None, stream=None):
    """Confidence of the listed masked rows and the unmasking of n_t of them
    (fdl_confidence_unmask).  logits [B, m_max, V] fp32 or bf16 (last axis contiguous),
    pos [B, m_max] int32 ascending; mask [B, L] uint8 and conf [B, L] fp32 are updated in
    place; tokens [B, L] int32 or None.  Returns unmasked [B, n_t] int32 (or None)."""
    if logits.dim() != 3 or logits.stride(2) != 1:
        raise FdlError(2, "logits must be [B, m_max, V] with a contiguous last axis")
    B, m_max, V = logits.shape
    L = mask.shape[1]
    for name, t, dt in (("pos", pos, torch.int32), ("mask", mask, torch.uint8), ("conf", conf, torch.float32)):
        if t.dtype != dt or not t.is_contiguous():
            raise FdlError(2, f"{name} must be a contiguous {dt} tensor")
    if tokens is not None and (tokens.dtype != torch.int32 or not tokens.is_contiguous()):
        raise FdlError(2, "tokens must be a contiguous int32 [B, L] tensor")
    if unmasked is None and want_unmasked:
        unmasked = torch.empty((B, max(n_t, 1)), dtype=torch.int32, device=logits.device)
    nbytes = int(lib().fdl_confidence_unmask_workspace_bytes(B, V, m_max))
    ws, ws_n = _ws(workspace, logits.device).get(nbytes)
    st = lib().fdl_confidence_unmask(_dtype_code(logits), B, L, V, _ptr(logits),
                                     Strides(logits.stride(0), 0, logits.stride(1)), _ptr(pos), _ptr(n_rows), m_max,
                                     int(n_t), _ptr(mask), _ptr(conf), _ptr(tokens), _ptr(unmasked), ws, ws_n,
                                     _stream(stream))
    _check(st, "fdl_confidence_unmask")
    return None if unmasked is None else unmasked[:, :n_t]


def dcu_select(x_now, x_prev, key_tokens, w_m: int, total: int, *, out=None, workspace=None, stream=None):
    """Per-layer cache update sets of the dynamic cache update (fdl_dcu_select).
    x_now, x_prev [B, NL, L, H] fp32 or bf16 (last axis contiguous); key_tokens [B, n_keys]
    int32 (entries outside [0, L) ignored) or None.  Returns (dist [B, NL, L] fp32,
    activity [B, NL] fp64, budgets [B, NL] int32, upd_idx [B, NL, L] int32, n_upd [B, NL]
    int32); the update set of (b, l) is upd_idx[b, l, :n_upd[b, l]].  `out` may hold those five
    tensors to write into."""
    if x_now.dim() != 4 or x_now.shape != x_prev.shape or x_now.dtype != x_prev.dtype:
        raise FdlError(2, "x_now and x_prev must be [B, NL, L, H] tensors of one shape and dtype")
    if x_now.stride(3) != 1 or x_prev.stride(3) != 1:
        raise FdlError(2, "x_now and x_prev need a contiguous last axis")
    B, NL, L, H = x_now.shape
    dev = x_now.device
    if key_tokens is not None and (key_tokens.dtype != torch.int32 or not key_tokens.is_contiguous()
                                   or key_tokens.dim() != 2 or key_tokens.shape[0] != B):
        raise FdlError(2, "key_tokens must be a contiguous int32 [B, n_keys] tensor")
    n_keys = 0 if key_tokens is None else key_tokens.shape[1]
    if out is None:
        out = (torch.empty((B, NL, L), dtype=torch.float32, device=dev),
               torch.empty((B, NL), dtype=torch.float64, device=dev),
               torch.empty((B, NL), dtype=torch.int32, device=dev),
               torch.empty((B, NL, L), dtype=torch.int32, device=dev),
               torch.empty((B, NL), dtype=torch.int32, device=dev))
    dist, activity, budgets, upd_idx, n_upd = out
    for name, t, dt in (("dist", dist, torch.float32), ("activity", activity, torch.float64),
                        ("budgets", budgets, torch.int32), ("upd_idx", upd_idx, torch.int32),
                        ("n_upd", n_upd, torch.int32)):
        if t.dtype != dt or not t.is_contiguous():
            raise FdlError(2, f"{name} must be a contiguous {dt} tensor")
    nbytes = int(lib().fdl_dcu_select_workspace_bytes(B, NL, L))
    ws, ws_n = _ws(workspace, dev).get(nbytes)
    xs = [Strides(t.stride(0), t.stride(1), t.stride(2)) for t in (x_now, x_prev)]
    st = lib().fdl_dcu_select(_dtype_code(x_now), B, NL, L, H, _ptr(x_now), xs[0], _ptr(x_prev), xs[1],
                              _ptr(key_tokens), n_keys, int(w_m), int(total), _ptr(dist), _ptr(activity),
                              _ptr(budgets), _ptr(upd_idx), _ptr(n_upd), ws, ws_n, _stream(stream))
    _check(st, "fdl_dcu_select")
    return dist, activity, budgets, upd_idx, n_upd


def calibrate_read(x: torch.Tensor, workgroups: int, *, sink=None, stream=None):
    """Streams the bytes of the contiguous device tensor x once (fdl_calibrate_read) and
    returns the [workgroups] int32 tensor of per-workgroup XORs of its 32-bit words."""
    if not x.is_contiguous() or (x.numel() * x.element_size()) % 16:
        raise FdlError(2, "x must be contiguous with a size that is a multiple of 16 bytes")
    if sink is None:
        sink = torch.empty((workgroups,), dtype=torch.int32, device=x.device)
    st = lib().fdl_calibrate_read(_ptr(x), x.numel() * x.element_size(), _ptr(sink), int(workgroups),
                                  _stream(stream))
    _check(st, "fdl_calibrate_read")
    return sink


def calibrate_mfma(workgroups: int, iters: int, a_val: float, b_val: float, *, device="cuda", sink=None,
                   stream=None):
    """Back-to-back bf16 MFMAs on register operands (fdl_calibrate_mfma); returns the
    [workgroups * 4, 2] fp32 tensor of per-wave (accumulator element, largest deviation)."""
    if sink is None:
        sink = torch.empty((workgroups * 4, 2), dtype=torch.float32, device=device)
    st = lib().fdl_calibrate_mfma(int(workgroups), int(iters), float(a_val), float(b_val), _ptr(sink),
                                  _stream(stream))
    _check(st, "fdl_calibrate_mfma")
    return sink


CALIBRATE_MFMA_FLOPS_PER_WAVE_ROUND = 8 * 2 * 32 * 32 * 16

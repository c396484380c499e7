"""ctypes binding of libnsa (the C ABI declared in include/nsa.h).

Argument marshalling only: every step of NSA runs in the library's HIP
kernels.  Torch tensors supply device memory; calls are enqueued on torch's
current stream.  If the library is missing the import of any entry point
raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .config import BF16, FP32, NSAShape

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnsa.so")

(OP_FORWARD, OP_SELECT, OP_DECODE, OP_SPARSE, OP_BACKWARD, OP_DSA_DECODE, OP_DSA_PREFILL, OP_BACKWARD_MLP,
 OP_CMP_WINDOW) = range(9)
STATUS = {0: "NSA_OK", -1: "NSA_ERR_NULL", -2: "NSA_ERR_SHAPE", -3: "NSA_ERR_DTYPE", -4: "NSA_ERR_PARAM",
          -5: "NSA_ERR_WORKSPACE", -6: "NSA_ERR_HIP", -7: "NSA_ERR_ALIGN"}

EXPORTS = ("nsa_workspace_bytes", "nsa_compress_kv", "nsa_compress_kv_mlp", "nsa_compress_append", "nsa_compress_append_mlp", "nsa_compressed_attention",
           "nsa_compressed_window_attention", "nsa_select_topn",
           "nsa_sparse_attention", "nsa_pack_kv_blocks", "nsa_window_attention", "nsa_selected_attention", "nsa_select_blocks",
           "nsa_forward", "nsa_forward_train", "nsa_decode_step", "nsa_decode_step_noalloc", "nsa_backward", "nsa_backward_mlp", "nsa_dsa_decode", "nsa_dsa_prefill", "nsa_status_string")


class NSAError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__("%s: %s (%d): %s" % (fn, STATUS.get(status, "?"), status, msg))
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "H_kv", "group", "d_k", "d_v", "l", "d", "l_sel", "n",
                                              "w")] + [("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """Load libnsa.so (built by ``python -m sparse_attention_long_07_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libnsa.so is not built (%s); run python -m sparse_attention_long_07_amd.build"
                              % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.nsa_workspace_bytes.restype = ctypes.c_size_t
        L.nsa_workspace_bytes.argtypes = [ctypes.POINTER(Config), ctypes.c_int]
        L.nsa_status_string.restype = ctypes.c_char_p
        L.nsa_status_string.argtypes = [ctypes.c_int]
        L.nsa_compress_kv.restype = ctypes.c_int
        L.nsa_compress_kv.argtypes = [ctypes.POINTER(Config)] + [_vp] * 9
        L.nsa_dsa_decode.restype = ctypes.c_int
        L.nsa_dsa_decode.argtypes = ([ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                                     + [_vp] * 10 + [_vp, ctypes.c_size_t, _vp])
        L.nsa_dsa_prefill.restype = ctypes.c_int
        L.nsa_dsa_prefill.argtypes = ([ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                                      + [_vp] * 9 + [_vp, ctypes.c_size_t, _vp])
        L.nsa_compress_kv_mlp.restype = ctypes.c_int
        L.nsa_compress_kv_mlp.argtypes = [ctypes.POINTER(Config)] + [_vp] * 11
        L.nsa_compress_append.restype = ctypes.c_int
        L.nsa_compress_append.argtypes = [ctypes.POINTER(Config), _vp, _vp, ctypes.c_int32] + [_vp] * 9
        L.nsa_compress_append_mlp.restype = ctypes.c_int
        L.nsa_compress_append_mlp.argtypes = [ctypes.POINTER(Config), _vp, _vp, ctypes.c_int32] + [_vp] * 11
        L.nsa_compressed_attention.restype = ctypes.c_int
        L.nsa_compressed_attention.argtypes = [ctypes.POINTER(Config)] + [_vp] * 6
        L.nsa_compressed_window_attention.restype = ctypes.c_int
        L.nsa_compressed_window_attention.argtypes = [ctypes.POINTER(Config)] + [_vp] * 11 + [ctypes.c_size_t, _vp]
        L.nsa_select_topn.restype = ctypes.c_int
        L.nsa_select_topn.argtypes = [ctypes.POINTER(Config)] + [_vp] * 3
        L.nsa_sparse_attention.restype = ctypes.c_int
        L.nsa_sparse_attention.argtypes = [ctypes.POINTER(Config)] + [_vp] * 9 + [ctypes.c_size_t, _vp]
        L.nsa_pack_kv_blocks.restype = ctypes.c_int
        L.nsa_pack_kv_blocks.argtypes = [ctypes.POINTER(Config), _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.nsa_window_attention.restype = ctypes.c_int
        L.nsa_window_attention.argtypes = [ctypes.POINTER(Config)] + [_vp] * 8
        L.nsa_selected_attention.restype = ctypes.c_int
        L.nsa_selected_attention.argtypes = [ctypes.POINTER(Config)] + [_vp] * 8 + [ctypes.c_size_t, _vp]
        L.nsa_select_blocks.restype = ctypes.c_int
        L.nsa_select_blocks.argtypes = [ctypes.POINTER(Config), _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.nsa_forward.restype = ctypes.c_int
        L.nsa_forward.argtypes = [ctypes.POINTER(Config)] + [_vp] * 12 + [ctypes.c_size_t, _vp]
        L.nsa_forward_train.restype = ctypes.c_int
        L.nsa_forward_train.argtypes = [ctypes.POINTER(Config)] + [_vp] * 14 + [ctypes.c_size_t, _vp]
        L.nsa_decode_step.restype = ctypes.c_int
        L.nsa_decode_step.argtypes = [ctypes.POINTER(Config)] + [_vp] * 12 + [ctypes.c_size_t, _vp]
        L.nsa_decode_step_noalloc.restype = ctypes.c_int
        L.nsa_decode_step_noalloc.argtypes = [ctypes.POINTER(Config)] + [_vp] * 12
        L.nsa_backward.restype = ctypes.c_int
        L.nsa_backward.argtypes = [ctypes.POINTER(Config)] + [_vp] * 25 + [ctypes.c_size_t, _vp]
        L.nsa_backward_mlp.restype = ctypes.c_int
        L.nsa_backward_mlp.argtypes = [ctypes.POINTER(Config)] + [_vp] * 29 + [ctypes.c_size_t, _vp]
        _lib = L
    return _lib


def config(s: NSAShape, scale: float = 0.0) -> Config:
    return Config(s.B, s.T, s.Hkv, s.G, s.dk, s.dv, s.l, s.d, s.lsel, s.n, s.w, scale,
                  0 if s.dtype == FP32 else 1)


def _check(fn, st):
    if st != 0:
        raise NSAError(fn, st, lib().nsa_status_string(st).decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(s: NSAShape):
    return torch.bfloat16 if s.dtype == BF16 else torch.float32


def _req(t, name, shape, dtype):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError("%s: expected contiguous %s %s, got %s %s" % (name, tuple(shape), dtype,
                                                                       tuple(t.shape), t.dtype))
    return t


def workspace_bytes(s: NSAShape, op: int) -> int:
    return int(lib().nsa_workspace_bytes(ctypes.byref(config(s)), op))


def workspace(s: NSAShape, op: int, device="cuda") -> torch.Tensor:
    """A workspace tensor for `op` (torch's allocator returns 256-byte aligned memory)."""
    return torch.empty(max(1, workspace_bytes(s, op)), dtype=torch.uint8, device=device)


def compress_kv(s: NSAShape, k, v, w_ck, pe_k, w_cv, pe_v, cmp_k=None, cmp_v=None):
    dt = _dt(s)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(w_ck, "w_ck", (s.dk, s.l * s.dk), dt)
    _req(pe_k, "pe_k", (s.l, s.dk), dt)
    _req(w_cv, "w_cv", (s.dv, s.l * s.dv), dt)
    _req(pe_v, "pe_v", (s.l, s.dv), dt)
    if cmp_k is None:
        cmp_k = torch.empty((s.B, s.Hkv, s.n_pad, s.dk), dtype=dt, device=k.device)
    if cmp_v is None:
        cmp_v = torch.empty((s.B, s.Hkv, s.n_pad, s.dv), dtype=dt, device=k.device)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    c = config(s)
    _check("nsa_compress_kv", lib().nsa_compress_kv(ctypes.byref(c), _p(k), _p(v), _p(w_ck), _p(pe_k), _p(w_cv),
                                                    _p(pe_v), _p(cmp_k), _p(cmp_v), _stream()))
    return cmp_k, cmp_v


def compress_kv_mlp(s: NSAShape, k, v, w1_k, pe_k, w2_k, w1_v, pe_v, w2_v, cmp_k=None, cmp_v=None):
    """Two-layer compression: cmp = W2 relu(W1 vec(block + PE)) for K and V."""
    dt = _dt(s)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(w1_k, "w1_k", (s.dk, s.l * s.dk), dt)
    _req(pe_k, "pe_k", (s.l, s.dk), dt)
    _req(w2_k, "w2_k", (s.dk, s.dk), dt)
    _req(w1_v, "w1_v", (s.dv, s.l * s.dv), dt)
    _req(pe_v, "pe_v", (s.l, s.dv), dt)
    _req(w2_v, "w2_v", (s.dv, s.dv), dt)
    if cmp_k is None:
        cmp_k = torch.empty((s.B, s.Hkv, s.n_pad, s.dk), dtype=dt, device=k.device)
    if cmp_v is None:
        cmp_v = torch.empty((s.B, s.Hkv, s.n_pad, s.dv), dtype=dt, device=k.device)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    c = config(s)
    _check("nsa_compress_kv_mlp",
           lib().nsa_compress_kv_mlp(ctypes.byref(c), _p(k), _p(v), _p(w1_k), _p(pe_k), _p(w2_k), _p(w1_v),
                                     _p(pe_v), _p(w2_v), _p(cmp_k), _p(cmp_v), _stream()))
    return cmp_k, cmp_v


def compress_append(s: NSAShape, len_old, len_new, max_append, k_cache, v_cache, w_ck, pe_k, w_cv, pe_v, cmp_k,
                    cmp_v):
    """Compressed entries of the blocks that growing each cache from len_old[b]
    to len_new[b] tokens completes (s.T = cache capacity; len_old may be None
    for all zero).  cmp_k / cmp_v are updated in place and returned."""
    dt = _dt(s)
    if len_old is not None:
        _req(len_old, "len_old", (s.B,), torch.int32)
    _req(len_new, "len_new", (s.B,), torch.int32)
    _req(k_cache, "k_cache", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v_cache, "v_cache", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(w_ck, "w_ck", (s.dk, s.l * s.dk), dt)
    _req(pe_k, "pe_k", (s.l, s.dk), dt)
    _req(w_cv, "w_cv", (s.dv, s.l * s.dv), dt)
    _req(pe_v, "pe_v", (s.l, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    c = config(s)
    _check("nsa_compress_append",
           lib().nsa_compress_append(ctypes.byref(c), _p(len_old), _p(len_new), int(max_append), _p(k_cache),
                                     _p(v_cache), _p(w_ck), _p(pe_k), _p(w_cv), _p(pe_v), _p(cmp_k), _p(cmp_v),
                                     _stream()))
    return cmp_k, cmp_v


def compress_append_mlp(s: NSAShape, len_old, len_new, max_append, k_cache, v_cache, w1_k, pe_k, w2_k, w1_v, pe_v,
                        w2_v, cmp_k, cmp_v):
    """compress_append with the two-layer map of compress_kv_mlp.  cmp_k /
    cmp_v are updated in place and returned."""
    dt = _dt(s)
    if len_old is not None:
        _req(len_old, "len_old", (s.B,), torch.int32)
    _req(len_new, "len_new", (s.B,), torch.int32)
    _req(k_cache, "k_cache", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v_cache, "v_cache", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(w1_k, "w1_k", (s.dk, s.l * s.dk), dt)
    _req(pe_k, "pe_k", (s.l, s.dk), dt)
    _req(w2_k, "w2_k", (s.dk, s.dk), dt)
    _req(w1_v, "w1_v", (s.dv, s.l * s.dv), dt)
    _req(pe_v, "pe_v", (s.l, s.dv), dt)
    _req(w2_v, "w2_v", (s.dv, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    c = config(s)
    _check("nsa_compress_append_mlp",
           lib().nsa_compress_append_mlp(ctypes.byref(c), _p(len_old), _p(len_new), int(max_append), _p(k_cache),
                                         _p(v_cache), _p(w1_k), _p(pe_k), _p(w2_k), _p(w1_v), _p(pe_v), _p(w2_v),
                                         _p(cmp_k), _p(cmp_v), _stream()))
    return cmp_k, cmp_v


def compressed_attention(s: NSAShape, q, cmp_k, cmp_v=None, o_cmp=None, scores=None):
    """Stage S2: returns (o_cmp, scores); o_cmp is None when cmp_v is None."""
    dt = _dt(s)
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    if cmp_v is not None:
        _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
        if o_cmp is None:
            o_cmp = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=q.device)
        _req(o_cmp, "o_cmp", (s.B, s.T, s.Hq, s.dv), dt)
    else:
        o_cmp = None
    if scores is None:
        scores = torch.empty((s.B, s.Hkv, s.T, s.nb), dtype=torch.float32, device=q.device)
    _req(scores, "scores", (s.B, s.Hkv, s.T, s.nb), torch.float32)
    c = config(s)
    _check("nsa_compressed_attention", lib().nsa_compressed_attention(ctypes.byref(c), _p(q), _p(cmp_k), _p(cmp_v),
                                                                      _p(o_cmp), _p(scores), _stream()))
    return o_cmp, scores


def compressed_window_attention(s: NSAShape, q, k, v, cmp_k, cmp_v, w_g, b_g, scores=None, o=None, o_cmp=None,
                                ws=None):
    """Stage S2 and the window half of S4 in one call: returns (o, scores),
    o = g_cmp o_cmp + g_win o_win; o_cmp is written only when given."""
    dt = _dt(s)
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    if scores is None:
        scores = torch.empty((s.B, s.Hkv, s.T, s.nb), dtype=torch.float32, device=q.device)
    _req(scores, "scores", (s.B, s.Hkv, s.T, s.nb), torch.float32)
    if o is None:
        o = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=q.device)
    _req(o, "o", (s.B, s.T, s.Hq, s.dv), dt)
    if o_cmp is not None:
        _req(o_cmp, "o_cmp", (s.B, s.T, s.Hq, s.dv), dt)
    if ws is None and o_cmp is None and workspace_bytes(s, OP_CMP_WINDOW) > 0:
        ws = workspace(s, OP_CMP_WINDOW, q.device)
    c = config(s)
    _check("nsa_compressed_window_attention",
           lib().nsa_compressed_window_attention(ctypes.byref(c), _p(q), _p(k), _p(v), _p(cmp_k), _p(cmp_v), _p(w_g),
                                                 _p(b_g), _p(scores), _p(o), _p(o_cmp), _p(ws),
                                                 0 if ws is None else ws.numel(), _stream()))
    return o, scores


def select_topn(s: NSAShape, scores, idx=None):
    """Stage S3: idx [B,Hkv,T,n] from scores [B,Hkv,T,nb]."""
    _req(scores, "scores", (s.B, s.Hkv, s.T, s.nb), torch.float32)
    if idx is None:
        idx = torch.empty((s.B, s.Hkv, s.T, s.n), dtype=torch.int32, device=scores.device)
    _req(idx, "idx", (s.B, s.Hkv, s.T, s.n), torch.int32)
    c = config(s)
    _check("nsa_select_topn", lib().nsa_select_topn(ctypes.byref(c), _p(scores), _p(idx), _stream()))
    return idx


def sparse_attention(s: NSAShape, q, k, v, o_cmp, idx, w_g, b_g, o=None, ws=None):
    """Stage S4: selected + window attention and the gated sum."""
    dt = _dt(s)
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(o_cmp, "o_cmp", (s.B, s.T, s.Hq, s.dv), dt)
    _req(idx, "idx", (s.B, s.Hkv, s.T, s.n), torch.int32)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    if o is None:
        o = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=q.device)
    _req(o, "o", (s.B, s.T, s.Hq, s.dv), dt)
    if ws is None:
        ws = workspace(s, OP_SPARSE, q.device)
    c = config(s)
    _check("nsa_sparse_attention", lib().nsa_sparse_attention(ctypes.byref(c), _p(q), _p(k), _p(v), _p(o_cmp),
                                                              _p(idx), _p(w_g), _p(b_g), _p(o), _p(ws), ws.numel(),
                                                              _stream()))
    return o


def pack_kv_blocks(s: NSAShape, k, v, ws=None):
    """K and V repacked per 64-token block for selected_attention; returns
    the workspace that holds them (empty on shapes that read K/V directly)."""
    dt = _dt(s)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    if ws is None:
        ws = workspace(s, OP_SPARSE, k.device)
    c = config(s)
    _check("nsa_pack_kv_blocks", lib().nsa_pack_kv_blocks(ctypes.byref(c), _p(k), _p(v), _p(ws), ws.numel(),
                                                          _stream()))
    return ws


def window_attention(s: NSAShape, q, k, v, o_cmp, w_g, b_g, o=None):
    """Window half of stage S4: o = g_cmp o_cmp + g_win o_win."""
    dt = _dt(s)
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(o_cmp, "o_cmp", (s.B, s.T, s.Hq, s.dv), dt)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    if o is None:
        o = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=q.device)
    _req(o, "o", (s.B, s.T, s.Hq, s.dv), dt)
    c = config(s)
    _check("nsa_window_attention", lib().nsa_window_attention(ctypes.byref(c), _p(q), _p(k), _p(v), _p(o_cmp),
                                                              _p(w_g), _p(b_g), _p(o), _stream()))
    return o


def selected_attention(s: NSAShape, q, k, v, idx, w_g, b_g, o, ws):
    """Selected half of stage S4: o += g_slc o_slc (o updated in place);
    ws is what pack_kv_blocks returned for the same k and v."""
    dt = _dt(s)
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(idx, "idx", (s.B, s.Hkv, s.T, s.n), torch.int32)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    _req(o, "o", (s.B, s.T, s.Hq, s.dv), dt)
    c = config(s)
    _check("nsa_selected_attention", lib().nsa_selected_attention(ctypes.byref(c), _p(q), _p(k), _p(v), _p(idx),
                                                                   _p(w_g), _p(b_g), _p(o), _p(ws), ws.numel(),
                                                                   _stream()))
    return o


def select_blocks(s: NSAShape, q, cmp_k, want_scores=False, idx_out=None, ws=None):
    dt = _dt(s)
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    scores = torch.empty((s.B, s.Hkv, s.T, s.nb), dtype=torch.float32, device=q.device) if want_scores else None
    if idx_out is None:
        idx_out = torch.empty((s.B, s.Hkv, s.T, s.n), dtype=torch.int32, device=q.device)
    _req(idx_out, "idx_out", (s.B, s.Hkv, s.T, s.n), torch.int32)
    if ws is None:
        ws = workspace(s, OP_SELECT, q.device)
    c = config(s)
    _check("nsa_select_blocks", lib().nsa_select_blocks(ctypes.byref(c), _p(q), _p(cmp_k), _p(scores),
                                                        _p(idx_out), _p(ws), ws.numel(), _stream()))
    return (idx_out, scores) if want_scores else idx_out


def forward(s: NSAShape, q, k, v, cmp_k, cmp_v, w_g, b_g, idx_in=None, o=None, want_idx=False,
            want_scores=False, ws=None):
    """NSA prefill forward; returns o (and idx / scores if asked)."""
    dt = _dt(s)
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    if idx_in is not None:
        _req(idx_in, "idx_in", (s.B, s.Hkv, s.T, s.n), torch.int32)
    if o is None:
        o = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=q.device)
    _req(o, "o", (s.B, s.T, s.Hq, s.dv), dt)
    idx = torch.empty((s.B, s.Hkv, s.T, s.n), dtype=torch.int32, device=q.device) if want_idx else None
    scores = torch.empty((s.B, s.Hkv, s.T, s.nb), dtype=torch.float32, device=q.device) if want_scores else None
    if ws is None:
        ws = workspace(s, OP_FORWARD, q.device)
    c = config(s)
    _check("nsa_forward", lib().nsa_forward(ctypes.byref(c), _p(q), _p(k), _p(v), _p(cmp_k), _p(cmp_v), _p(w_g),
                                            _p(b_g), _p(idx_in), _p(o), _p(idx), _p(scores), _p(ws), ws.numel(),
                                            _stream()))
    out = [o]
    if want_idx:
        out.append(idx)
    if want_scores:
        out.append(scores)
    return out[0] if len(out) == 1 else tuple(out)


def forward_train(s: NSAShape, q, k, v, cmp_k, cmp_v, w_g, b_g, idx_in=None, o=None, want_idx=False, ws=None):
    """forward() that also saves each branch's softmax statistics for the
    backward.  Returns o and saved = (lse [3,B,T,Hq] fp32, o_branch
    [3,B,T,Hq,dv] config dtype), then idx if asked: (o, saved[, idx])."""
    dt = _dt(s)
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    if idx_in is not None:
        _req(idx_in, "idx_in", (s.B, s.Hkv, s.T, s.n), torch.int32)
    if o is None:
        o = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=q.device)
    _req(o, "o", (s.B, s.T, s.Hq, s.dv), dt)
    idx = torch.empty((s.B, s.Hkv, s.T, s.n), dtype=torch.int32, device=q.device) if want_idx else None
    lse = torch.empty((3, s.B, s.T, s.Hq), dtype=torch.float32, device=q.device)
    obr = torch.empty((3, s.B, s.T, s.Hq, s.dv), dtype=dt, device=q.device)
    if ws is None:
        ws = workspace(s, OP_FORWARD, q.device)
    c = config(s)
    _check("nsa_forward_train",
           lib().nsa_forward_train(ctypes.byref(c), _p(q), _p(k), _p(v), _p(cmp_k), _p(cmp_v), _p(w_g), _p(b_g),
                                   _p(idx_in), _p(o), _p(idx), None, _p(lse), _p(obr), _p(ws), ws.numel(),
                                   _stream()))
    return (o, (lse, obr), idx) if want_idx else (o, (lse, obr))


def _saved_ptrs(s: NSAShape, saved, dt):
    """Pointers of a forward_train `saved` pair, or two NULLs."""
    if saved is None:
        return None, None
    lse, obr = saved
    _req(lse, "lse_saved", (3, s.B, s.T, s.Hq), torch.float32)
    _req(obr, "o_saved", (3, s.B, s.T, s.Hq, s.dv), dt)
    return _p(lse), _p(obr)


def decode_step(s: NSAShape, seq_lens, q, k_cache, v_cache, cmp_k, cmp_v, w_g, b_g, idx_in=None, o=None,
                want_idx=False, ws=None):
    """One decode step (s.T = cache capacity); returns o [B,Hq,dv] (and idx [B,Hkv,n])."""
    dt = _dt(s)
    _req(seq_lens, "seq_lens", (s.B,), torch.int32)
    _req(q, "q", (s.B, s.Hq, s.dk), dt)
    _req(k_cache, "k_cache", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v_cache, "v_cache", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    if idx_in is not None:
        _req(idx_in, "idx_in", (s.B, s.Hkv, s.n), torch.int32)
    if o is None:
        o = torch.empty((s.B, s.Hq, s.dv), dtype=dt, device=q.device)
    _req(o, "o", (s.B, s.Hq, s.dv), dt)
    idx = torch.empty((s.B, s.Hkv, s.n), dtype=torch.int32, device=q.device) if want_idx else None
    if ws is None:
        ws = workspace(s, OP_DECODE, q.device)
    c = config(s)
    _check("nsa_decode_step", lib().nsa_decode_step(ctypes.byref(c), _p(seq_lens), _p(q), _p(k_cache),
                                                    _p(v_cache), _p(cmp_k), _p(cmp_v), _p(w_g), _p(b_g),
                                                    _p(idx_in), _p(o), _p(idx), _p(ws), ws.numel(), _stream()))
    return (o, idx) if want_idx else o


def decode_step_noalloc(s: NSAShape, seq_lens, q, k_cache, v_cache, cmp_k, cmp_v, w_g, b_g, idx_in=None, o=None,
                        want_idx=False):
    """decode_step with the library's own static scratch as the workspace
    (nsa_decode_step_noalloc: no allocation by the library)."""
    dt = _dt(s)
    _req(seq_lens, "seq_lens", (s.B,), torch.int32)
    _req(q, "q", (s.B, s.Hq, s.dk), dt)
    _req(k_cache, "k_cache", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v_cache, "v_cache", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    if idx_in is not None:
        _req(idx_in, "idx_in", (s.B, s.Hkv, s.n), torch.int32)
    if o is None:
        o = torch.empty((s.B, s.Hq, s.dv), dtype=dt, device=q.device)
    _req(o, "o", (s.B, s.Hq, s.dv), dt)
    idx = torch.empty((s.B, s.Hkv, s.n), dtype=torch.int32, device=q.device) if want_idx else None
    c = config(s)
    _check("nsa_decode_step_noalloc",
           lib().nsa_decode_step_noalloc(ctypes.byref(c), _p(seq_lens), _p(q), _p(k_cache), _p(v_cache), _p(cmp_k),
                                         _p(cmp_v), _p(w_g), _p(b_g), _p(idx_in), _p(o), _p(idx), _stream()))
    return (o, idx) if want_idx else o


def dsa_decode(s: NSAShape, idx_heads, idx_dim, topk, seq_lens, q_idx, w_idx, k_idx, q, k_cache, v_cache,
               sel_in=None, sel=None, o=None, ws=None):
    """DSA-style decode step (s.T = cache capacity): indexer scores, top-k
    token selection (skipped with sel_in) and attention over the selected
    tokens.  Returns (sel [B,topk] int32 or sel_in, o [B,Hq,dv])."""
    dt = _dt(s)
    dev = q.device
    _req(seq_lens, "seq_lens", (s.B,), torch.int32)
    _req(q, "q", (s.B, s.Hq, s.dk), dt)
    _req(k_cache, "k_cache", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v_cache, "v_cache", (s.B, s.Hkv, s.T, s.dv), dt)
    if sel_in is not None:
        _req(sel_in, "sel_in", (s.B, topk), torch.int32)
    else:
        _req(q_idx, "q_idx", (s.B, idx_heads, idx_dim), dt)
        _req(w_idx, "w_idx", (s.B, idx_heads), dt)
        _req(k_idx, "k_idx", (s.B, s.T, idx_dim), dt)
        if sel is None:
            sel = torch.empty((s.B, topk), dtype=torch.int32, device=dev)
        _req(sel, "sel", (s.B, topk), torch.int32)
        if ws is None:
            ws = workspace(s, OP_DSA_DECODE, dev)
    if o is None:
        o = torch.empty((s.B, s.Hq, s.dv), dtype=dt, device=dev)
    _req(o, "o", (s.B, s.Hq, s.dv), dt)
    c = config(s)
    _check("nsa_dsa_decode", lib().nsa_dsa_decode(ctypes.byref(c), idx_heads, idx_dim, topk, _p(seq_lens), _p(q_idx),
                                                  _p(w_idx), _p(k_idx), _p(q), _p(k_cache), _p(v_cache),
                                                  _p(sel_in), _p(sel), _p(o), _p(ws),
                                                  0 if ws is None else ws.numel(), _stream()))
    return (sel_in if sel_in is not None else sel), o


def dsa_prefill(s: NSAShape, idx_heads, idx_dim, topk, q_idx, w_idx, k_idx, q, k, v, sel_in=None, sel=None, o=None,
                ws=None):
    """DSA-style attention for every position: indexer scores, top-k tokens
    per position (skipped with sel_in) and attention over them.  Returns
    (sel [B,T,topk] int32 or sel_in, o [B,T,Hq,dv])."""
    dt = _dt(s)
    dev = q.device
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    if sel_in is not None:
        _req(sel_in, "sel_in", (s.B, s.T, topk), torch.int32)
    else:
        _req(q_idx, "q_idx", (s.B, s.T, idx_heads, idx_dim), dt)
        _req(w_idx, "w_idx", (s.B, s.T, idx_heads), dt)
        _req(k_idx, "k_idx", (s.B, s.T, idx_dim), dt)
        if sel is None:
            sel = torch.empty((s.B, s.T, topk), dtype=torch.int32, device=dev)
        _req(sel, "sel", (s.B, s.T, topk), torch.int32)
        if ws is None:
            ws = workspace(s, OP_DSA_PREFILL, dev)
    if o is None:
        o = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=dev)
    _req(o, "o", (s.B, s.T, s.Hq, s.dv), dt)
    c = config(s)
    _check("nsa_dsa_prefill", lib().nsa_dsa_prefill(ctypes.byref(c), idx_heads, idx_dim, topk, _p(q_idx), _p(w_idx),
                                                    _p(k_idx), _p(q), _p(k), _p(v), _p(sel_in), _p(sel), _p(o),
                                                    _p(ws), 0 if ws is None else ws.numel(), _stream()))
    return (sel_in if sel_in is not None else sel), o


def backward(s: NSAShape, q, k, v, cmp_k, cmp_v, w_ck, pe_k, w_cv, pe_v, w_g, b_g, idx, d_o, ws=None,
             saved=None):
    """Gradients of sum(d_o * o) with the selection idx held fixed.  Returns a
    dict d_q, d_k, d_v (config dtype) and d_wck, d_pek, d_wcv, d_pev, d_wg,
    d_bg (fp32), in the layouts of the corresponding inputs.  saved: the
    (lse, o_branch) pair forward_train returned for these inputs, or None."""
    dt = _dt(s)
    dev = q.device
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    _req(w_ck, "w_ck", (s.dk, s.l * s.dk), dt)
    _req(pe_k, "pe_k", (s.l, s.dk), dt)
    _req(w_cv, "w_cv", (s.dv, s.l * s.dv), dt)
    _req(pe_v, "pe_v", (s.l, s.dv), dt)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    _req(idx, "idx", (s.B, s.Hkv, s.T, s.n), torch.int32)
    _req(d_o, "d_o", (s.B, s.T, s.Hq, s.dv), dt)
    g = {"d_q": torch.empty_like(q), "d_k": torch.empty_like(k), "d_v": torch.empty_like(v),
         "d_wck": torch.empty(w_ck.shape, dtype=torch.float32, device=dev),
         "d_pek": torch.empty(pe_k.shape, dtype=torch.float32, device=dev),
         "d_wcv": torch.empty(w_cv.shape, dtype=torch.float32, device=dev),
         "d_pev": torch.empty(pe_v.shape, dtype=torch.float32, device=dev),
         "d_wg": torch.empty(w_g.shape, dtype=torch.float32, device=dev),
         "d_bg": torch.empty(b_g.shape, dtype=torch.float32, device=dev)}
    if ws is None:
        ws = workspace(s, OP_BACKWARD, dev)
    c = config(s)
    st = lib().nsa_backward(ctypes.byref(c), _p(q), _p(k), _p(v), _p(cmp_k), _p(cmp_v), _p(w_ck), _p(pe_k),
                            _p(w_cv), _p(pe_v), _p(w_g), _p(b_g), _p(idx), _p(d_o),
                            *[_p(g[n]) for n in ("d_q", "d_k", "d_v", "d_wck", "d_pek", "d_wcv", "d_pev", "d_wg",
                                                 "d_bg")],
                            *_saved_ptrs(s, saved, dt), _p(ws), ws.numel(), _stream())
    _check("nsa_backward", st)
    return g


def backward_mlp(s: NSAShape, q, k, v, cmp_k, cmp_v, w1_k, pe_k, w2_k, w1_v, pe_v, w2_v, w_g, b_g, idx, d_o,
                 ws=None, saved=None):
    """backward() with the two-layer compression map (compress_kv_mlp).
    Returns a dict d_q, d_k, d_v (config dtype) and d_w1k, d_pek, d_w2k,
    d_w1v, d_pev, d_w2v, d_wg, d_bg (fp32), in the layouts of the inputs."""
    dt = _dt(s)
    dev = q.device
    _req(q, "q", (s.B, s.T, s.Hq, s.dk), dt)
    _req(k, "k", (s.B, s.Hkv, s.T, s.dk), dt)
    _req(v, "v", (s.B, s.Hkv, s.T, s.dv), dt)
    _req(cmp_k, "cmp_k", (s.B, s.Hkv, s.n_pad, s.dk), dt)
    _req(cmp_v, "cmp_v", (s.B, s.Hkv, s.n_pad, s.dv), dt)
    _req(w1_k, "w1_k", (s.dk, s.l * s.dk), dt)
    _req(pe_k, "pe_k", (s.l, s.dk), dt)
    _req(w2_k, "w2_k", (s.dk, s.dk), dt)
    _req(w1_v, "w1_v", (s.dv, s.l * s.dv), dt)
    _req(pe_v, "pe_v", (s.l, s.dv), dt)
    _req(w2_v, "w2_v", (s.dv, s.dv), dt)
    _req(w_g, "w_g", (s.Hq, 3, s.dk), dt)
    _req(b_g, "b_g", (s.Hq, 3), dt)
    _req(idx, "idx", (s.B, s.Hkv, s.T, s.n), torch.int32)
    _req(d_o, "d_o", (s.B, s.T, s.Hq, s.dv), dt)
    f32 = lambda t: torch.empty(t.shape, dtype=torch.float32, device=dev)
    g = {"d_q": torch.empty_like(q), "d_k": torch.empty_like(k), "d_v": torch.empty_like(v),
         "d_w1k": f32(w1_k), "d_pek": f32(pe_k), "d_w2k": f32(w2_k), "d_w1v": f32(w1_v), "d_pev": f32(pe_v),
         "d_w2v": f32(w2_v), "d_wg": f32(w_g), "d_bg": f32(b_g)}
    if ws is None:
        ws = workspace(s, OP_BACKWARD_MLP, dev)
    c = config(s)
    st = lib().nsa_backward_mlp(ctypes.byref(c), _p(q), _p(k), _p(v), _p(cmp_k), _p(cmp_v), _p(w1_k), _p(pe_k),
                                _p(w2_k), _p(w1_v), _p(pe_v), _p(w2_v), _p(w_g), _p(b_g), _p(idx), _p(d_o),
                                *[_p(g[n]) for n in ("d_q", "d_k", "d_v", "d_w1k", "d_pek", "d_w2k", "d_w1v", "d_pev",
                                                     "d_w2v", "d_wg", "d_bg")],
                                *_saved_ptrs(s, saved, dt), _p(ws), ws.numel(), _stream())
    _check("nsa_backward_mlp", st)
    return g

"""Python access to the NSA CPU oracle (``nsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  All arrays are
float64 numpy arrays; inputs stored in bf16 or fp32 convert to float64 exactly.

The C library is built with gcc (``-O2``, no fast-math, so the compiler keeps
the source's summation order) on first use or by :func:`build`.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_nsa.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/liboracle_nsa.so``."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "T", "Hkv", "G", "dk", "dv", "l", "d", "lsel", "n", "w")] + [
        ("scale", ctypes.c_double)]


_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.orc_n_cmp.restype = ctypes.c_int
        lib.orc_n_cmp.argtypes = [ctypes.c_int] * 3
        lib.orc_round_bf16.restype = ctypes.c_double
        lib.orc_round_bf16.argtypes = [ctypes.c_double]
        lib.orc_compress.restype = None
        lib.orc_compress.argtypes = [ctypes.c_int] * 8 + [_dp, _dp, _dp, _dp]
        lib.orc_compress_mlp.restype = None
        lib.orc_compress_mlp.argtypes = [ctypes.c_int] * 8 + [_dp] * 5
        lib.orc_forward_rows.restype = None
        lib.orc_forward_rows.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int, _ip, _ip, _dp, _dp, _dp,
                                         ctypes.c_int, _dp, _dp, _dp, _dp, _ip, _dp, _ip, _dp, ctypes.c_int,
                                         _dp, _dp]
        lib.orc_backward.restype = None
        lib.orc_backward.argtypes = [ctypes.POINTER(_Cfg)] + [_dp] * 9 + [_ip, _dp, ctypes.c_int] + [_dp] * 9
        lib.orc_backward_mlp.restype = None
        lib.orc_backward_mlp.argtypes = [ctypes.POINTER(_Cfg)] + [_dp] * 11 + [_ip, _dp, ctypes.c_int] + [_dp] * 11
        lib.orc_select.restype = ctypes.c_int
        lib.orc_select.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int, _dp, _ip]
        _lib = lib
    return _lib


@dataclass
class Cfg:
    """Shape and method parameters of one call (defaults: the pages' values)."""
    B: int
    T: int
    Hkv: int
    G: int
    dk: int
    dv: int
    l: int = 32
    d: int = 16
    lsel: int = 64
    n: int = 16
    w: int = 512
    scale: float | None = None

    @property
    def Hq(self) -> int:
        return self.Hkv * self.G

    @property
    def nb(self) -> int:
        """Selection blocks covering the sequence."""
        return -(-self.T // self.lsel)

    def c(self) -> _Cfg:
        s = self.scale if self.scale is not None else 1.0 / math.sqrt(self.dk)
        return _Cfg(self.B, self.T, self.Hkv, self.G, self.dk, self.dv, self.l, self.d, self.lsel, self.n,
                    self.w, s)


def _d(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


def _i(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_ip)


def n_cmp(T: int, l: int = 32, d: int = 16) -> int:
    return _load().orc_n_cmp(T, l, d)


def round_bf16(x: float) -> float:
    return _load().orc_round_bf16(float(x))


def compress(x, W, PE, l: int = 32, d: int = 16, n_out: int | None = None, round_bf16: bool = False):
    """x [B,H,T,dim], W [dim, l*dim], PE [l, dim] -> [B,H,n_out,dim]."""
    x, xp = _d(x)
    B, H, T, dim = x.shape
    W, wp = _d(W)
    PE, pp = _d(PE)
    assert W.shape == (dim, l * dim) and PE.shape == (l, dim)
    if n_out is None:
        n_out = n_cmp(T, l, d)
    out = np.zeros((B, H, n_out, dim))
    _load().orc_compress(B, H, T, dim, l, d, n_out, int(round_bf16), xp, wp, pp, out.ctypes.data_as(_dp))
    return out


def compress_mlp(x, W1, PE, W2, l: int = 32, d: int = 16, n_out: int | None = None, round_bf16: bool = False):
    """Two-layer compression: x [B,H,T,dim], W1 [dim, l*dim], PE [l, dim],
    W2 [dim, dim] -> [B,H,n_out,dim] = W2 relu(W1 vec(block + PE)), the hidden
    layer and the output rounded to bf16 when round_bf16."""
    x, xp = _d(x)
    B, H, T, dim = x.shape
    W1, w1p = _d(W1)
    PE, pp = _d(PE)
    W2, w2p = _d(W2)
    assert W1.shape == (dim, l * dim) and PE.shape == (l, dim) and W2.shape == (dim, dim)
    if n_out is None:
        n_out = n_cmp(T, l, d)
    out = np.zeros((B, H, n_out, dim))
    _load().orc_compress_mlp(B, H, T, dim, l, d, n_out, int(round_bf16), xp, w1p, pp, w2p, out.ctypes.data_as(_dp))
    return out


def forward_rows(cfg: Cfg, b_list, t_list, q_rows, kc, vc, k, v, wg, bg, idx_in=None,
                 want_scores=False, want_branches=False, want_lse=False):
    """NSA forward for the listed rows.

    q_rows [R, Hq, dk] (row r = position t_list[r] of batch b_list[r]);
    kc [B,Hkv,npad,dk], vc [B,Hkv,npad,dv]; k [B,Hkv,T,dk], v [B,Hkv,T,dv];
    wg [Hq,3,dk], bg [Hq,3]; idx_in [R,Hkv,n] or None.
    Returns dict with o [R,Hq,dv], idx [R,Hkv,n] and optionally
    scores [R,Hkv,nb], branches [R,3,Hq,dv] (o_cmp, o_slc, o_win) and lse
    [R,3,Hq] (each branch's log-sum-exp of its logits, -inf when empty).
    """
    assert cfg.n <= 64
    b_arr, bp = _i(b_list)
    t_arr, tp = _i(t_list)
    R = int(b_arr.shape[0])
    q_rows, qp = _d(q_rows)
    kc, kcp = _d(kc)
    vc, vcp = _d(vc)
    k, kp = _d(k)
    v, vp = _d(v)
    wg, wgp = _d(wg)
    bg, bgp = _d(bg)
    assert q_rows.shape == (R, cfg.Hq, cfg.dk)
    assert k.shape == (cfg.B, cfg.Hkv, cfg.T, cfg.dk) and v.shape == (cfg.B, cfg.Hkv, cfg.T, cfg.dv)
    npad = kc.shape[2]
    assert kc.shape == (cfg.B, cfg.Hkv, npad, cfg.dk) and vc.shape == (cfg.B, cfg.Hkv, npad, cfg.dv)
    assert npad >= n_cmp(int(t_arr.max()) + 1 if R else 0, cfg.l, cfg.d)
    assert wg.shape == (cfg.Hq, 3, cfg.dk) and bg.shape == (cfg.Hq, 3)
    assert R == 0 or (0 <= int(t_arr.min()) and int(t_arr.max()) < cfg.T)
    if idx_in is not None:
        idx_in, iip = _i(idx_in)
        assert idx_in.shape == (R, cfg.Hkv, cfg.n)
    else:
        iip = None
    o = np.zeros((R, cfg.Hq, cfg.dv))
    idx = np.zeros((R, cfg.Hkv, cfg.n), dtype=np.int32)
    nb = cfg.nb
    scores = np.zeros((R, cfg.Hkv, nb)) if want_scores else None
    branches = np.zeros((R, 3, cfg.Hq, cfg.dv)) if want_branches else None
    lse = np.zeros((R, 3, cfg.Hq)) if want_lse else None
    c = cfg.c()
    _load().orc_forward_rows(ctypes.byref(c), R, bp, tp, qp, kcp, vcp, npad, kp, vp, wgp, bgp, iip,
                             o.ctypes.data_as(_dp), idx.ctypes.data_as(_ip),
                             scores.ctypes.data_as(_dp) if want_scores else None, nb,
                             branches.ctypes.data_as(_dp) if want_branches else None,
                             lse.ctypes.data_as(_dp) if want_lse else None)
    out = {"o": o, "idx": idx}
    if want_scores:
        out["scores"] = scores
    if want_branches:
        out["branches"] = branches
    if want_lse:
        out["lse"] = lse
    return out


def forward(cfg: Cfg, q, kc, vc, k, v, wg, bg, idx_in=None, **kw):
    """Whole prefill forward.  q [B,T,Hq,dk]; idx_in [B,Hkv,T,n] or None.

    Returns o [B,T,Hq,dv], idx [B,Hkv,T,n] and the optional extras of
    :func:`forward_rows` reshaped to [B,T,...] (scores to [B,Hkv,T,nb])."""
    q = np.asarray(q)
    B, T = cfg.B, cfg.T
    bl = np.repeat(np.arange(B), T)
    tl = np.tile(np.arange(T), B)
    ii = None
    if idx_in is not None:
        ii = np.asarray(idx_in).transpose(0, 2, 1, 3).reshape(B * T, cfg.Hkv, cfg.n)
    r = forward_rows(cfg, bl, tl, q.reshape(B * T, cfg.Hq, cfg.dk), kc, vc, k, v, wg, bg, ii, **kw)
    out = {"o": r["o"].reshape(B, T, cfg.Hq, cfg.dv),
           "idx": r["idx"].reshape(B, T, cfg.Hkv, cfg.n).transpose(0, 2, 1, 3).copy()}
    if "scores" in r:
        out["scores"] = r["scores"].reshape(B, T, cfg.Hkv, -1).transpose(0, 2, 1, 3).copy()
    if "branches" in r:
        out["branches"] = r["branches"].reshape(B, T, 3, cfg.Hq, cfg.dv)
    if "lse" in r:
        out["lse"] = r["lse"].reshape(B, T, 3, cfg.Hq)
    return out


def decode(cfg: Cfg, seq_lens, q, kc, vc, k, v, wg, bg, idx_in=None):
    """Decode step: q [B,Hq,dk] is the query of the last cached token of each
    sequence (t = seq_lens[b]-1); caches k [B,Hkv,T,dk] etc. with T = capacity.
    Returns o [B,Hq,dv], idx [B,Hkv,n]."""
    seq = np.asarray(seq_lens, dtype=np.int32)
    assert seq.shape == (cfg.B,) and int(seq.min()) >= 1 and int(seq.max()) <= cfg.T
    r = forward_rows(cfg, np.arange(cfg.B), seq - 1, q, kc, vc, k, v, wg, bg, idx_in)
    return {"o": r["o"], "idx": r["idx"]}


def select(cfg: Cfg, t: int, S):
    """Selection for one row from given scores S[0..t//lsel]."""
    S, sp = _d(S)
    assert S.shape[0] >= t // cfg.lsel + 1
    idx = np.zeros(cfg.n, dtype=np.int32)
    c = cfg.c()
    _load().orc_select(ctypes.byref(c), t, sp, idx.ctypes.data_as(_ip))
    return idx


def backward(cfg: Cfg, q, k, v, wck, pek, wcv, pev, wg, bg, idx, dO, round_bf16: bool = False):
    """Gradients of L = sum(dO * o) with the selection idx [B,Hkv,T,n] held
    fixed.  q [B,T,Hq,dk], k [B,Hkv,T,dk], v [B,Hkv,T,dv], wck [dk,l*dk],
    pek [l,dk], wcv [dv,l*dv], pev [l,dv], wg [Hq,3,dk], bg [Hq,3],
    dO [B,T,Hq,dv].  The compressed K/V are recomputed from k/v (rounded to
    bf16 when round_bf16, the rounding passed straight through in reverse).
    Returns dict dq, dk, dv, dwck, dpek, dwcv, dpev, dwg, dbg (input layouts).
    Rows whose dO is zero for all heads of a KV group are skipped (their
    contribution is exactly zero)."""
    B, T, Hkv, Hq, dk, dv, l = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.dk, cfg.dv, cfg.l
    arrs = []
    for a, shp in ((q, (B, T, Hq, dk)), (k, (B, Hkv, T, dk)), (v, (B, Hkv, T, dv)), (wck, (dk, l * dk)),
                   (pek, (l, dk)), (wcv, (dv, l * dv)), (pev, (l, dv)), (wg, (Hq, 3, dk)), (bg, (Hq, 3))):
        a, _ = _d(a)
        assert a.shape == shp, (a.shape, shp)
        arrs.append(a)
    idx, ip = _i(idx)
    assert idx.shape == (B, Hkv, T, cfg.n)
    dO, dop = _d(dO)
    assert dO.shape == (B, T, Hq, dv)
    out = {"dq": np.zeros((B, T, Hq, dk)), "dk": np.zeros((B, Hkv, T, dk)), "dv": np.zeros((B, Hkv, T, dv)),
           "dwck": np.zeros((dk, l * dk)), "dpek": np.zeros((l, dk)), "dwcv": np.zeros((dv, l * dv)),
           "dpev": np.zeros((l, dv)), "dwg": np.zeros((Hq, 3, dk)), "dbg": np.zeros((Hq, 3))}
    c = cfg.c()
    _load().orc_backward(ctypes.byref(c), *[a.ctypes.data_as(_dp) for a in arrs], ip, dop, int(round_bf16),
                         *[out[n].ctypes.data_as(_dp) for n in ("dq", "dk", "dv", "dwck", "dpek", "dwcv",
                                                                 "dpev", "dwg", "dbg")])
    return out


def backward_mlp(cfg: Cfg, q, k, v, w1k, pek, w2k, w1v, pev, w2v, wg, bg, idx, dO, round_bf16: bool = False):
    """backward() with the two-layer compression map of compress_mlp for K
    and V: w1k [dk,l*dk], pek [l,dk], w2k [dk,dk], w1v [dv,l*dv], pev [l,dv],
    w2v [dv,dv].  Returns dict dq, dk, dv, dw1k, dpek, dw2k, dw1v, dpev, dw2v,
    dwg, dbg (input layouts); the hidden layer and the compressed K/V are
    recomputed (rounded to bf16 when round_bf16, the roundings passed straight
    through in reverse)."""
    B, T, Hkv, Hq, dk, dv, l = cfg.B, cfg.T, cfg.Hkv, cfg.Hq, cfg.dk, cfg.dv, cfg.l
    arrs = []
    for a, shp in ((q, (B, T, Hq, dk)), (k, (B, Hkv, T, dk)), (v, (B, Hkv, T, dv)), (w1k, (dk, l * dk)),
                   (pek, (l, dk)), (w2k, (dk, dk)), (w1v, (dv, l * dv)), (pev, (l, dv)), (w2v, (dv, dv)),
                   (wg, (Hq, 3, dk)), (bg, (Hq, 3))):
        a, _ = _d(a)
        assert a.shape == shp, (a.shape, shp)
        arrs.append(a)
    idx, ip = _i(idx)
    assert idx.shape == (B, Hkv, T, cfg.n)
    dO, dop = _d(dO)
    assert dO.shape == (B, T, Hq, dv)
    names = ("dq", "dk", "dv", "dw1k", "dpek", "dw2k", "dw1v", "dpev", "dw2v", "dwg", "dbg")
    shapes = ((B, T, Hq, dk), (B, Hkv, T, dk), (B, Hkv, T, dv), (dk, l * dk), (l, dk), (dk, dk), (dv, l * dv),
              (l, dv), (dv, dv), (Hq, 3, dk), (Hq, 3))
    out = {n: np.zeros(sh) for n, sh in zip(names, shapes)}
    c = cfg.c()
    _load().orc_backward_mlp(ctypes.byref(c), *[a.ctypes.data_as(_dp) for a in arrs], ip, dop, int(round_bf16),
                             *[out[n].ctypes.data_as(_dp) for n in names])
    return out

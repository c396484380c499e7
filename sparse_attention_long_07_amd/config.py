"""NSA problem shapes, the named workloads, and algorithmic work accounting.

The method parameters default to the values given on valuable12.com,
"AI 모델의 '긴 문장 처리' 한계 돌파, 딥시크의 새 어텐션 기술 화제", section II:
compression block l=32, stride d=16, selection block l'=64, n=16 selected
blocks (including the initial block and 2 local blocks), window w=512.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

FP32 = "fp32"
BF16 = "bf16"


@dataclass(frozen=True)
class NSAShape:
    B: int
    T: int
    Hkv: int
    G: int
    dk: int
    dv: int
    dtype: str = BF16
    l: int = 32
    d: int = 16
    lsel: int = 64
    n: int = 16
    w: int = 512

    @property
    def Hq(self) -> int:
        return self.Hkv * self.G

    @property
    def n_cmp(self) -> int:
        """Complete compression blocks of a length-T sequence."""
        return 0 if self.T < self.l else (self.T - self.l) // self.d + 1

    @property
    def n_pad(self) -> int:
        """Compressed slots allocated per (batch, KV head): N_cmp rounded up to 64."""
        return max(64, -(-self.n_cmp // 64) * 64)

    @property
    def nb(self) -> int:
        """Selection blocks covering the sequence."""
        return -(-self.T // self.lsel)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)

    @property
    def esize(self) -> int:
        return 4 if self.dtype == FP32 else 2

    def with_(self, **kw) -> "NSAShape":
        return replace(self, **kw)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: NSAShape
    kind: str            # "prefill", "decode" or "fwdbwd"
    unit_scaled: bool    # inputs ~ N(0,1)/sqrt(fan_in) when True, N(0,1) otherwise
    description: str


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fp32_T1024", NSAShape(1, 1024, 1, 4, 64, 64, FP32), "prefill", True,
                 "NSA forward fp32, B=1, T=1024 causal, 1 KV head x 4 query heads, d_k=d_v=64"),
        Workload("bf16_T8192", NSAShape(1, 8192, 4, 16, 192, 128), "prefill", True,
                 "NSA prefill forward bf16, B=1, T=8192, 4 KV heads x 16 query heads, d_k=192, d_v=128"),
        Workload("bf16_T65536", NSAShape(1, 65536, 4, 16, 192, 128), "prefill", False,
                 "NSA prefill forward bf16, B=1, T=65536, 4 KV groups x 16 query heads, d_k=192, d_v=128"),
        Workload("bf16_decode_B32_T65536", NSAShape(32, 65536, 4, 16, 192, 128), "decode", False,
                 "NSA decode step bf16, 32 sequences with 65,536-token caches, 4 KV groups x 16 query heads"),
        Workload("bf16_fwdbwd_T16384", NSAShape(1, 16384, 4, 16, 192, 128), "fwdbwd", False,
                 "NSA forward+backward bf16, B=1, T=16384, 4 KV groups x 16 query heads, d_k=192, d_v=128"),
    ]
}


# ---------------------------------------------------------------------------
# Algorithmic work.  Only causal-visible keys are counted; QK^T and PV cost
# 2*(d_k + d_v) flops per (query head, key).  Exponentials, masked keys, pad
# slots and any recomputation are not counted.

def _visible_cmp(t: int, s: NSAShape) -> int:
    return (t - (s.l - 1)) // s.d + 1 if t >= s.l - 1 else 0


def _selected_tokens(t: int, s: NSAShape) -> int:
    jcur = t // s.lsel
    nsel = min(s.n, jcur + 1)      # the current block is always among them
    return (nsel - 1) * s.lsel + (t - jcur * s.lsel + 1)


def row_key_counts(t: int, s: NSAShape) -> tuple[int, int, int]:
    """(compressed, selected, window) keys one query position attends to."""
    return _visible_cmp(t, s), _selected_tokens(t, s), min(s.w, t + 1)


def prefill_flops(s: NSAShape) -> dict:
    """Algorithmic flops of one prefill forward, by branch."""
    per_key = 2 * (s.dk + s.dv) * s.Hq * s.B
    cmp = slc = win = 0
    # closed forms are easy to get wrong at block edges; a loop over t is exact
    # and takes well under a second even at T=65536
    for t in range(s.T):
        a, b, c = row_key_counts(t, s)
        cmp += a
        slc += b
        win += c
    compress = 2 * s.n_cmp * s.l * (s.dk * s.dk + s.dv * s.dv) * s.Hkv * s.B
    gates = 2 * 3 * s.dk * s.Hq * s.T * s.B
    out = {"compressed": cmp * per_key, "selected": slc * per_key, "window": win * per_key,
           "compress": compress, "gates": gates}
    out["total"] = sum(out.values())
    return out


def backward_flops(s: NSAShape) -> dict:
    """Algorithmic flops of one backward pass with the selection held fixed.

    Per attended (query head, key) pair of a branch the gradient takes five
    products: the scores again (d_k), dP = dO V^T (d_v), dV (d_v), dK (d_k)
    and dq (d_k), i.e. 2 (3 d_k + 2 d_v) flops against 2 (d_k + d_v) forward.
    The compression map's backward is two products per forward one (dW and
    the token gradient), the gates' likewise (dW_g and the dq term)."""
    f = prefill_flops(s)
    ratio = (3 * s.dk + 2 * s.dv) / (s.dk + s.dv)
    attn = (f["compressed"] + f["selected"] + f["window"]) * ratio
    out = {"attention": int(attn), "compress": 2 * f["compress"], "gates": 2 * f["gates"]}
    out["total"] = sum(out.values())
    return out


def dense_causal_flops(s: NSAShape) -> int:
    """Flops of full causal attention at the same shape (for the pages' speedup context)."""
    return s.T * (s.T + 1) // 2 * 2 * (s.dk + s.dv) * s.Hq * s.B


def decode_slots(s: NSAShape) -> dict:
    """Key slots one decode step reads per (sequence, KV group) at t = T-1.

    The compressed cache is read in whole 64-slot tiles, so at T=65536 the
    4,095 valid compressed entries occupy 4,096 slots; with 16 selected
    blocks of 64 and a 512-token window that is the 5,632 tokens reported for
    64k decoding (valuable12.com, section III.3)."""
    t = s.T - 1
    cmp_valid = _visible_cmp(t, s)
    cmp_slots = -(-cmp_valid // 64) * 64
    sel = min(s.n, t // s.lsel + 1) * s.lsel
    win = min(s.w, t + 1)
    return {"cmp_valid": cmp_valid, "cmp_slots": cmp_slots, "selected": sel, "window": win,
            "total_slots": cmp_slots + sel + win}


def decode_bytes(s: NSAShape) -> int:
    """Algorithmic HBM bytes of one decode step: K and V rows of every slot read."""
    per_slot = (s.dk + s.dv) * s.esize
    return decode_slots(s)["total_slots"] * per_slot * s.B * s.Hkv


def decode_flops(s: NSAShape) -> int:
    t = s.T - 1
    a, b, c = row_key_counts(t, s)
    return (a + b + c) * 2 * (s.dk + s.dv) * s.Hq * s.B

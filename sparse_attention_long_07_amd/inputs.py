"""Seeded synthetic inputs for NSA.

This module only draws random numbers and casts them to the storage dtype; it
holds none of the method's arithmetic.  It is the one module that both the
HIP path (tests, benchmark) and the CPU oracle's callers share.

Recipe (draw order fixed: q, k, v, W_ck, PE_k, W_cv, PE_v, W_g, b_g, dO):
  * activations q, k ~ N(0,1)/sqrt(d_k), v ~ N(0,1)/sqrt(d_v) for the
    unit-scaled workloads, plain N(0,1) otherwise;
  * W_ck ~ N(0,1)/sqrt(l*d_k), W_cv ~ N(0,1)/sqrt(l*d_v), W_g ~ N(0,1)/sqrt(d_k);
  * PE_k, b_g ~ N(0,1)/sqrt(d_k), PE_v ~ N(0,1)/sqrt(d_v);
  * dO ~ N(0,1).
Values are drawn in float32 with a torch generator on the target device and
then cast (round to nearest even) to the workload dtype.  Tests that compare
with the oracle copy the device tensors to the host, so both sides always see
identical values.
"""
from __future__ import annotations

import math

import torch

from .config import BF16, NSAShape


def torch_dtype(s: NSAShape) -> torch.dtype:
    return torch.bfloat16 if s.dtype == BF16 else torch.float32


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, std, gen, device, dtype):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_weights(s: NSAShape, gen, device, dtype):
    return {
        "w_ck": _randn((s.dk, s.l * s.dk), 1 / math.sqrt(s.l * s.dk), gen, device, dtype),
        "pe_k": _randn((s.l, s.dk), 1 / math.sqrt(s.dk), gen, device, dtype),
        "w_cv": _randn((s.dv, s.l * s.dv), 1 / math.sqrt(s.l * s.dv), gen, device, dtype),
        "pe_v": _randn((s.l, s.dv), 1 / math.sqrt(s.dv), gen, device, dtype),
        "w_g": _randn((s.Hq, 3, s.dk), 1 / math.sqrt(s.dk), gen, device, dtype),
        "b_g": _randn((s.Hq, 3), 1 / math.sqrt(s.dk), gen, device, dtype),
    }


def make_mlp_weights(s: NSAShape, seed: int, device="cpu", nonneg: bool = False):
    """Second-layer weights of the two-layer compression map, drawn in this
    order: W2_k ~ N(0,1)/sqrt(d_k) [d_k, d_k], W2_v ~ N(0,1)/sqrt(d_v) [d_v, d_v]
    (absolute values when nonneg).  The first layer and PE use the linear
    map's tensors (W_ck, PE_k, W_cv, PE_v), whose shapes it shares."""
    g = _gen(seed, device)
    dt = torch_dtype(s)
    w2k = _randn((s.dk, s.dk), 1 / math.sqrt(s.dk), g, device, dt)
    w2v = _randn((s.dv, s.dv), 1 / math.sqrt(s.dv), g, device, dt)
    if nonneg:
        w2k, w2v = w2k.abs(), w2v.abs()
    return {"w2_k": w2k, "w2_v": w2v}


def make_dsa_indexer(s: NSAShape, seed: int, device="cpu", idx_heads: int = 4, idx_dim: int = 64):
    """Indexer inputs of a DSA-style decode step, drawn in this order:
    q_idx ~ N(0,1)/sqrt(idx_dim) [B, idx_heads, idx_dim], w_idx ~ N(0,1)/sqrt(idx_heads)
    [B, idx_heads], k_idx ~ N(0,1) [B, T, idx_dim] (s.T = cache capacity)."""
    g = _gen(seed, device)
    dt = torch_dtype(s)
    return {"q_idx": _randn((s.B, idx_heads, idx_dim), 1 / math.sqrt(idx_dim), g, device, dt),
            "w_idx": _randn((s.B, idx_heads), 1 / math.sqrt(idx_heads), g, device, dt),
            "k_idx": _randn((s.B, s.T, idx_dim), 1.0, g, device, dt)}


def make_prefill(s: NSAShape, seed: int, device="cpu", unit_scaled: bool = True, with_grad: bool = False):
    """q [B,T,Hq,dk], k [B,Hkv,T,dk], v [B,Hkv,T,dv] plus the weights."""
    dt = torch_dtype(s)
    gen = _gen(seed, device)
    sq = 1 / math.sqrt(s.dk) if unit_scaled else 1.0
    sv = 1 / math.sqrt(s.dv) if unit_scaled else 1.0
    out = {
        "q": _randn((s.B, s.T, s.Hq, s.dk), sq, gen, device, dt),
        "k": _randn((s.B, s.Hkv, s.T, s.dk), sq, gen, device, dt),
        "v": _randn((s.B, s.Hkv, s.T, s.dv), sv, gen, device, dt),
    }
    out.update(make_weights(s, gen, device, dt))
    if with_grad:
        out["do"] = _randn((s.B, s.T, s.Hq, s.dv), 1.0, gen, device, dt)
    return out


def make_decode(s: NSAShape, seed: int, device="cpu", unit_scaled: bool = False, seq_lens=None):
    """Decode inputs: q [B,Hq,dk] (one new token per sequence), raw caches
    k [B,Hkv,T,dk], v [B,Hkv,T,dv] with T the cache capacity, the weights,
    and seq_lens [B] int32 (all T unless given)."""
    dt = torch_dtype(s)
    gen = _gen(seed, device)
    sq = 1 / math.sqrt(s.dk) if unit_scaled else 1.0
    sv = 1 / math.sqrt(s.dv) if unit_scaled else 1.0
    out = {
        "q": _randn((s.B, s.Hq, s.dk), sq, gen, device, dt),
        "k": _randn((s.B, s.Hkv, s.T, s.dk), sq, gen, device, dt),
        "v": _randn((s.B, s.Hkv, s.T, s.dv), sv, gen, device, dt),
    }
    out.update(make_weights(s, gen, device, dt))
    if seq_lens is None:
        seq_lens = [s.T] * s.B
    out["seq_lens"] = torch.tensor(seq_lens, dtype=torch.int32, device=device)
    return out

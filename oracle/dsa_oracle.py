"""Plain CPU reference of a DSA-style decode step: lightning indexer, top-k
token selection, attention over the selected tokens.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code
with the HIP library.  Arithmetic is numpy float64; numpy's matmul and sort
serve as library steps.

Source: DSA explainer (allinfo.ai.kr), section "쉽게 이해하기": an indexer
with several small heads whose key is shared by all heads scores every past
token by a weighted sum of ReLU dot products; a selector keeps the 2,048
highest-scoring positions for each query independently; attention then runs
at full precision over the selected tokens only, with the softmax
denominator summed over the selected set.

Readings where the page is silent (listed in the repository's design notes):
  - indexer inputs are given per step: q_idx [H_I][d_I] and weights w_idx
    [H_I] for the query, k_idx [T][d_I] per cached token (their projections
    are model weights outside this step); one selection per sequence, shared
    by every query head and KV group (the key is shared across heads);
  - candidates are the cached tokens s < seq_len (the query is the token at
    seq_len - 1, which attends to itself);
  - order: higher score first, the lower position on equal scores; fewer
    than k candidates: all are taken; the list is ascending, -1 padded;
  - attention: per query head h of KV group g = h // G, softmax over the
    selected s of scale * q_h . k_g(s), output sum p v_g(s).
"""
from __future__ import annotations

import numpy as np


def index_scores(q_idx, w_idx, k_idx, L: int) -> np.ndarray:
    """I[s] = sum_j w_j relu(q_j . k_s) for s < L; q_idx [H_I, d_I], w_idx
    [H_I], k_idx [T, d_I] -> [L]."""
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w_idx, dtype=np.float64)
    k = np.asarray(k_idx, dtype=np.float64)[:L]
    dots = k @ q.T                                   # [L, H_I]
    return np.maximum(dots, 0.0) @ w


def select_topk(scores: np.ndarray, topk: int) -> np.ndarray:
    """Ascending positions of the topk highest scores (ties: lower position
    first), -1 padded to topk."""
    L = scores.shape[0]
    order = np.lexsort((np.arange(L), -scores))      # by -score, then position
    keep = np.sort(order[:min(topk, L)])
    out = -np.ones(topk, dtype=np.int64)
    out[:keep.size] = keep
    return out


def attend(q, k, v, sel, G: int, scale: float) -> np.ndarray:
    """q [Hq, d_k], k [Hkv, T, d_k], v [Hkv, T, d_v], sel: positions (-1
    ignored) -> o [Hq, d_v]: per head, softmax over the selected tokens."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = np.asarray(sel)
    s = s[s >= 0]
    Hq = q.shape[0]
    o = np.zeros((Hq, v.shape[-1]))
    if s.size == 0:
        return o
    for h in range(Hq):
        g = h // G
        z = (k[g, s] @ q[h]) * scale
        p = np.exp(z - z.max())
        p /= p.sum()
        o[h] = p @ v[g, s]
    return o


def dsa_decode(q_idx, w_idx, k_idx, q, k, v, seq_lens, topk: int, G: int, scale: float, sel_in=None):
    """One decode step for B sequences.  q_idx [B, H_I, d_I], w_idx [B, H_I],
    k_idx [B, T, d_I], q [B, Hq, d_k], k [B, Hkv, T, d_k], v [B, Hkv, T, d_v],
    seq_lens [B].  Returns (sel [B, topk] int64, o [B, Hq, d_v]); with sel_in
    the indexer and selector are skipped."""
    B = len(seq_lens)
    sel = np.zeros((B, topk), dtype=np.int64)
    o = np.zeros((B, np.shape(q)[1], np.shape(v)[-1]))
    for b in range(B):
        L = int(seq_lens[b])
        if sel_in is None:
            sel[b] = select_topk(index_scores(q_idx[b], w_idx[b], k_idx[b], L), topk)
        else:
            sel[b] = np.asarray(sel_in[b])
        o[b] = attend(q[b], k[b], v[b], sel[b], G, scale)
    return sel, o


def dsa_prefill(q_idx, w_idx, k_idx, q, k, v, topk: int, G: int, scale: float, sel_in=None, rows=None):
    """Every position t of B sequences as a query over its tokens s <= t.
    q_idx [B, T, H_I, d_I], w_idx [B, T, H_I], k_idx [B, T, d_I], q [B, T, Hq,
    d_k], k [B, Hkv, T, d_k], v [B, Hkv, T, d_v].  rows: (b, t) pairs to
    compute (default all).  Returns {(b, t): (sel [topk], o [Hq, d_v])}."""
    B, T = np.shape(q)[0], np.shape(q)[1]
    rows = rows if rows is not None else [(b, t) for b in range(B) for t in range(T)]
    out = {}
    for b, t in rows:
        if sel_in is None:
            sel = select_topk(index_scores(q_idx[b][t], w_idx[b][t], k_idx[b], t + 1), topk)
        else:
            sel = np.asarray(sel_in[b][t])
        out[(b, t)] = (sel, attend(q[b][t], k[b], v[b], sel, G, scale))
    return out


"""Pins of the DSA decode oracle (oracle/dsa_oracle.py) against facts that do
not come from its own arithmetic: closed forms of the indexer, the top-k
property checked pair by pair, torch's scaled-dot-product attention with a
mask built from the selection, and the numbers the DSA page prints
(tests/golden/dsa_allinfo.json).  CPU only."""
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import dsa_oracle as dsa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_indexer_closed_forms():
    rng = np.random.default_rng(0)
    T, d = 300, 8
    k = rng.standard_normal((T, d))
    x = k[:, 0]
    # one head reading channel 0 with weight 1: relu of that channel
    q1 = np.zeros((1, d))
    q1[0, 0] = 1.0
    np.testing.assert_array_equal(dsa.index_scores(q1, [1.0], k, T), np.maximum(x, 0.0))
    # two heads of opposite sign, weights 2 and 3: the relu is per head,
    # before the weighted sum (a relu of the sum would give 2x - 3x where x>0)
    q2 = np.zeros((2, d))
    q2[0, 0], q2[1, 0] = 1.0, -1.0
    got = dsa.index_scores(q2, [2.0, 3.0], k, T)
    np.testing.assert_allclose(got, np.where(x > 0, 2 * x, -3 * x), rtol=0, atol=1e-15)
    # only the first L tokens are scored
    assert dsa.index_scores(q2, [2.0, 3.0], k, 17).shape == (17,)
    # linear in the weights
    q3 = rng.standard_normal((4, d))
    w1, w2 = rng.standard_normal(4), rng.standard_normal(4)
    np.testing.assert_allclose(dsa.index_scores(q3, w1 + w2, k, T),
                               dsa.index_scores(q3, w1, k, T) + dsa.index_scores(q3, w2, k, T), atol=1e-12)


def _check_topk(scores, sel, k):
    L = scores.size
    n = min(k, L)
    kept = sel[:n]
    assert np.all(sel[n:] == -1) and np.all(kept >= 0) and np.all(np.diff(kept) > 0)
    out = np.setdiff1d(np.arange(L), kept)
    for i in kept:
        for j in out:
            # every kept position outranks every dropped one
            assert scores[i] > scores[j] or (scores[i] == scores[j] and i < j)


def test_selector_is_a_top_k():
    rng = np.random.default_rng(1)
    for L, k in ((50, 7), (40, 40), (12, 30), (64, 1)):
        sc = rng.standard_normal(L)
        _check_topk(sc, dsa.select_topk(sc, k), k)
    # ties at the boundary go to the lower positions
    sc = np.array([0.0, 1.0, 1.0, 2.0, 1.0, 1.0, -1.0])
    sel = dsa.select_topk(sc, 3)
    assert list(sel) == [1, 2, 3]
    _check_topk(sc, sel, 3)


def test_attention_equals_masked_sdpa():
    rng = np.random.default_rng(2)
    Hkv, G, T, dk, dv = 2, 3, 90, 16, 8
    q = rng.standard_normal((Hkv * G, dk))
    k = rng.standard_normal((Hkv, T, dk))
    v = rng.standard_normal((Hkv, T, dv))
    sel = np.sort(rng.choice(T, 25, replace=False))
    selp = np.concatenate([sel, -np.ones(7, dtype=int)])
    scale = 1 / math.sqrt(dk)
    got = dsa.attend(q, k, v, selp, G, scale)
    mask = torch.zeros(T, dtype=torch.bool)
    mask[torch.from_numpy(sel)] = True
    for h in range(Hkv * G):
        g = h // G
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[h][None, None, None]),
                                             torch.from_numpy(k[g][None, None]), torch.from_numpy(v[g][None, None]),
                                             attn_mask=mask[None, None, None], scale=scale)
        np.testing.assert_allclose(got[h], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_short_cache_is_dense_attention():
    # seq_len <= k: every cached token is selected; the step is plain attention
    rng = np.random.default_rng(3)
    B, Hkv, G, T, dk, dv, dI, HI = 2, 1, 4, 40, 16, 16, 8, 3
    L = [30, 40]
    qi, wi, ki = rng.standard_normal((B, HI, dI)), rng.standard_normal((B, HI)), rng.standard_normal((B, T, dI))
    q, k, v = rng.standard_normal((B, Hkv * G, dk)), rng.standard_normal((B, Hkv, T, dk)), rng.standard_normal((B, Hkv, T, dv))
    sel, o = dsa.dsa_decode(qi, wi, ki, q, k, v, L, 64, G, 0.25)
    for b in range(B):
        assert list(sel[b][:L[b]]) == list(range(L[b])) and np.all(sel[b][L[b]:] == -1)
        for h in range(Hkv * G):
            ref = F.scaled_dot_product_attention(torch.from_numpy(q[b, h][None, None, None]),
                                                 torch.from_numpy(k[b, h // G, :L[b]][None, None]),
                                                 torch.from_numpy(v[b, h // G, :L[b]][None, None]), scale=0.25)
            np.testing.assert_allclose(o[b, h], ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-12)


def test_golden_page_numbers():
    g = json.load(open(os.path.join(GOLDEN, "dsa_allinfo.json")))
    share = 100.0 * g["selected_tokens"] / g["context_tokens"]
    assert round(share, 1) == g["selected_share_percent"]                       # 1.5625% -> 1.6%
    assert g["context_tokens"] // g["selected_tokens"] == g["sparse_vs_full_ops_ratio"]   # 64x


def test_prefill_rows_are_decode_steps_and_causal_below_k():
    # position t of a prefill is the decode step at seq_len t + 1 on the same
    # cache; positions with t + 1 <= k select everything: causal attention
    rng = np.random.default_rng(6)
    B, Hkv, G, T, dk, dv, HI, dI, k = 1, 2, 2, 50, 8, 8, 3, 8, 20
    qi, wi, ki = rng.standard_normal((B, T, HI, dI)), rng.standard_normal((B, T, HI)), rng.standard_normal((B, T, dI))
    q, kk, v = rng.standard_normal((B, T, Hkv * G, dk)), rng.standard_normal((B, Hkv, T, dk)), rng.standard_normal((B, Hkv, T, dv))
    out = dsa.dsa_prefill(qi, wi, ki, q, kk, v, k, G, 0.3)
    for t in (0, 7, 19, 20, 49):
        sel_d, o_d = dsa.dsa_decode(qi[:, t], wi[:, t], ki, q[:, t], kk, v, [t + 1], k, G, 0.3)
        assert np.array_equal(out[(0, t)][0], sel_d[0]) and np.allclose(out[(0, t)][1], o_d[0], rtol=0, atol=1e-14)
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    for h in range(Hkv * G):
        ref = F.scaled_dot_product_attention(torch.from_numpy(q[0, :, h][None, None]),
                                             torch.from_numpy(kk[0, h // G][None, None]),
                                             torch.from_numpy(v[0, h // G][None, None]), attn_mask=mask[None, None],
                                             scale=0.3)[0, 0].numpy()
        for t in range(k):
            np.testing.assert_allclose(out[(0, t)][1][h], ref[t], rtol=1e-12, atol=1e-12)

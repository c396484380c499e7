"""DSA-style decode step (nsa_dsa_decode) against the oracle (oracle/dsa_oracle.py).

Selection: the GPU scores in fp32, the oracle in fp64.  A token's score error
is bounded by eps_s = 2^-20 * sum_j |w_j| sum_e |q_je k_se| (fp32 products
and sums over at most 16 x 256 terms), so the GPU list must be a valid top-k
of the oracle's scores within 2 eps_s of the k-th score, and must equal the
oracle's list exactly when no score other than the k-th score's own value
lies that close to it (this includes exact ties, such as the zeros of the
ReLU, which both sides break toward the lower position).
Attention: with the oracle's selection injected, o within 2e-2 of max |o|
(the bf16 output rule)."""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as dsa
from sparse_attention_long_07_amd import nsa
from sparse_attention_long_07_amd.config import NSAShape, WORKLOADS
from sparse_attention_long_07_amd.inputs import make_decode, make_dsa_indexer
from tests.parity_util import np64, out_tol

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nsa.lib()


def _clamp_len(L, T):
    return min(max(int(L), 1), T)


def _check_selection(scores, q_idx, w_idx, k_idx, L, got, topk, where):
    n = min(topk, L)
    g = got[:n]
    assert np.all(got[n:] == -1), where
    assert np.all(g >= 0) and np.all(g < L) and np.all(np.diff(g) > 0), where
    eps = 2.0 ** -20 * (np.abs(k_idx[:L]) @ np.abs(q_idx).T) @ np.abs(w_idx)
    ref = dsa.select_topk(scores, topk)
    if L <= topk:
        assert np.array_equal(got, ref), where
        return True
    tk = np.sort(scores)[::-1][topk - 1]
    out = np.setdiff1d(np.arange(L), g)
    assert np.all(scores[g] >= tk - 2 * eps[g]), where
    assert np.all(scores[out] <= tk + 2 * eps[out]), where
    near = (np.abs(scores - tk) <= 2 * eps) & (scores != tk)
    if not near.any():
        assert np.array_equal(got, ref), where
        return True
    return bool(np.array_equal(got, ref))


def _run(s, seq_lens, topk, hi, di, seed):
    x = make_decode(s, seed, "cuda", seq_lens=seq_lens)
    ix = make_dsa_indexer(s, seed + 1, "cuda", hi, di)
    sel, o = nsa.dsa_decode(s, hi, di, topk, x["seq_lens"], ix["q_idx"], ix["w_idx"], ix["k_idx"], x["q"], x["k"],
                            x["v"])
    torch.cuda.synchronize()
    return x, ix, sel.cpu().numpy(), o


CASES = [
    # (name, shape, seq_lens, topk, indexer heads, indexer dim)
    ("d192_T3000_k512", NSAShape(4, 3000, 2, 16, 192, 128), [3000, 2049, 513, 700], 512, 4, 64),
    ("d192_T3000_k2048", NSAShape(3, 3000, 2, 16, 192, 128), [3000, 2500, 1000], 2048, 4, 64),
    ("d128_T1500_k300", NSAShape(2, 1500, 1, 16, 128, 128), [1500, 301], 300, 8, 32),
    ("d64_T900_k64", NSAShape(3, 900, 3, 16, 64, 64), [900, 65, 1], 64, 16, 128),
]


@pytest.mark.parametrize("name,s,lens,topk,hi,di", CASES, ids=[c[0] for c in CASES])
def test_dsa_decode_parity(name, s, lens, topk, hi, di):
    say("dsa decode", name, s, lens, topk, hi, di)
    x, ix, sel, o = _run(s, lens, topk, hi, di, 81)
    G, scale = s.G, 1 / math.sqrt(s.dk)
    qi, wi, ki = np64(ix["q_idx"]), np64(ix["w_idx"]), np64(ix["k_idx"])
    q, k, v = np64(x["q"]), np64(x["k"]), np64(x["v"])
    n_same = 0
    for b in range(s.B):
        L = _clamp_len(lens[b], s.T)
        sc = dsa.index_scores(qi[b], wi[b], ki[b], L)
        # the GPU's list is a valid top-k (and the oracle's own where no near-tie
        # decides); the output is the oracle's attention over that list on every row
        n_same += _check_selection(sc, qi[b], wi[b], ki[b], L, sel[b], topk, (name, b))
        ref = dsa.attend(q[b], k[b], v[b], sel[b], G, scale)
        assert np.abs(np64(o[b]) - ref).max() <= out_tol(s, ref), (name, b)
    assert n_same >= 1, name


def _split_ws(s, n):
    """A workspace that holds an n-way split's partial results: per (sequence,
    KV group, share) 16 maxima, 16 sums and 16 x d_v outputs in fp32."""
    return torch.empty(4 * s.B * s.Hkv * n * (32 + 16 * s.dv), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("split", [1, 2, 4], ids=["one_wg", "split2", "split4"])
@pytest.mark.parametrize("name,s,lens,topk,hi,di", CASES, ids=[c[0] for c in CASES])
def test_dsa_attention_with_injected_selection(name, s, lens, topk, hi, di, split):
    """The oracle's selection injected: attention parity independent of
    selection near-ties; with a workspace that holds an n-way split's partials
    each KV group's slots run as n shares merged afterwards."""
    say("dsa attention", name, s, lens, topk, "split", split)
    x = make_decode(s, 83, "cuda", seq_lens=lens)
    ix = make_dsa_indexer(s, 84, "cuda", hi, di)
    qi, wi, ki = np64(ix["q_idx"]), np64(ix["w_idx"]), np64(ix["k_idx"])
    ref_sel, ref_o = dsa.dsa_decode(qi, wi, ki, np64(x["q"]), np64(x["k"]), np64(x["v"]),
                                    [_clamp_len(L, s.T) for L in lens], topk, s.G, 1 / math.sqrt(s.dk))
    sel_in = torch.from_numpy(ref_sel.astype(np.int32)).cuda()
    _, o = nsa.dsa_decode(s, hi, di, topk, x["seq_lens"], None, None, None, x["q"], x["k"], x["v"], sel_in=sel_in,
                          ws=_split_ws(s, split) if split > 1 else None)
    torch.cuda.synchronize()
    got = np64(o)
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref_o).max() <= out_tol(s, ref_o), name


def test_dsa_decode_full_size_sampled():
    """32 sequences at 65,536-token caches (the NSA decode workload's shape),
    top-2,048 with 4 indexer heads of 64, as bench.py times it (selection
    into the workspace, then the four-way split attention reusing it): the
    selection of 4 sequences against the oracle, their output against the
    oracle's attention over the GPU's selection, and the output of every
    other sequence equal bit for bit to the split attention run with the same
    selection injected."""
    s = WORKLOADS["bf16_decode_B32_T65536"].shape
    say("dsa decode full size", s)
    lens = [s.T] * s.B
    x, ix, sel, o = _run(s, lens, 2048, 4, 64, 85)
    qi, wi, ki = np64(ix["q_idx"][:4]), np64(ix["w_idx"][:4]), np64(ix["k_idx"][:4])
    q, k, v = np64(x["q"][:4]), np64(x["k"][:4]), np64(x["v"][:4])
    scale = 1 / math.sqrt(s.dk)
    ref_sel = []
    for b in range(4):
        sc = dsa.index_scores(qi[b], wi[b], ki[b], s.T)
        _check_selection(sc, qi[b], wi[b], ki[b], s.T, sel[b], 2048, ("full", b))
        ref_sel.append(dsa.select_topk(sc, 2048))
        # the timed path's own output: the oracle's attention over the GPU's selection
        ref = dsa.attend(q[b], k[b], v[b], sel[b], s.G, scale)
        assert np.abs(np64(o[b]) - ref).max() <= out_tol(s, ref), ("own selection", b)
    ref_sel = np.stack(ref_sel)
    # the selection of every other sequence against the oracle's scores too
    QI, WI, KI = np64(ix["q_idx"]), np64(ix["w_idx"]), np64(ix["k_idx"])
    for b in range(4, s.B):
        sc = dsa.index_scores(QI[b], WI[b], KI[b], s.T)
        _check_selection(sc, QI[b], WI[b], KI[b], s.T, sel[b], 2048, ("full", b))
    sel_in = torch.full((s.B, 2048), -1, dtype=torch.int32, device="cuda")
    sel_in[:4] = torch.from_numpy(ref_sel.astype(np.int32)).cuda()
    sel_in[4:] = torch.from_numpy(sel[4:]).cuda()
    _, o2 = nsa.dsa_decode(s, 4, 64, 2048, x["seq_lens"], None, None, None, x["q"], x["k"], x["v"], sel_in=sel_in,
                           ws=_split_ws(s, 4))
    torch.cuda.synchronize()
    # same selection, same split kernels: the same bits
    assert torch.equal(o[4:], o2[4:])
    for b in range(4):
        ref = dsa.attend(q[b], k[b], v[b], ref_sel[b], s.G, scale)
        assert np.abs(np64(o2[b]) - ref).max() <= out_tol(s, ref), b


@pytest.mark.parametrize("T,ncls", [(3000, 5), (20000, 5), (40000, 5), (40000, 2), (70000, 5)])
def test_dsa_decode_selection_ties(T, ncls):
    """Selection with massive exact ties: every cached indexer key is one of
    `ncls` rows, so a sequence's scores take that many values (identical bits
    on the GPU, whose every key runs the same products) and the k-th score is
    shared by thousands of positions; the list must be exactly the oracle's,
    which takes the tied positions lowest first.  The capacities span the
    selector's register-cached forms (16, 32 and 64 scores per lane; with two
    classes of 20,000 the candidates overflow the LDS list and the full passes
    run) and its re-reading form (T above 65,536)."""
    s = NSAShape(2, T, 1, 16, 64, 64)
    say("dsa ties", s, ncls)
    hi, di, topk = 4, 64, 2048
    ix = make_dsa_indexer(s, 87, "cuda", hi, di)
    base = ix["k_idx"][:, :ncls].clone()
    reps = torch.arange(T, device="cuda") % ncls
    ix["k_idx"] = base[:, reps].contiguous()
    lens = [T, T // 2 + 7]
    x = make_decode(s, 88, "cuda", seq_lens=lens)
    sel, _ = nsa.dsa_decode(s, hi, di, topk, x["seq_lens"], ix["q_idx"], ix["w_idx"], ix["k_idx"], x["q"], x["k"],
                            x["v"])
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    qi, wi, ki = np64(ix["q_idx"]), np64(ix["w_idx"]), np64(ix["k_idx"])
    for b in range(s.B):
        L = lens[b]
        sc = dsa.index_scores(qi[b], wi[b], ki[b], L)
        vals = np.unique(sc)
        assert len(vals) <= ncls
        assert np.array_equal(sel[b], dsa.select_topk(sc, topk)), (T, b)


PREFILL = [
    ("d192_T700_k128_B1H2", NSAShape(1, 700, 2, 16, 192, 128), 128, 4, 64),
    ("d64_T300_k64_B2H1", NSAShape(2, 300, 1, 16, 64, 64), 64, 8, 32),
]


@pytest.mark.parametrize("name,s,topk,hi,di", PREFILL, ids=[c[0] for c in PREFILL])
def test_dsa_prefill_parity(name, s, topk, hi, di):
    """Every position a query: sampled positions' selections against the
    oracle (as in the decode test), each sampled position's output against the
    oracle's attention over the GPU's own list, and the
    attention of every sampled position with the oracle's selection
    injected for all positions."""
    say("dsa prefill", name, s, topk)
    g = torch.Generator(device="cuda").manual_seed(91)
    dt = torch.bfloat16
    qi = (torch.randn((s.B, s.T, hi, di), generator=g, device="cuda") / math.sqrt(di)).to(dt)
    wi = (torch.randn((s.B, s.T, hi), generator=g, device="cuda") / math.sqrt(hi)).to(dt)
    ki = torch.randn((s.B, s.T, di), generator=g, device="cuda").to(dt)
    q = torch.randn((s.B, s.T, s.Hq, s.dk), generator=g, device="cuda").to(dt)
    k = torch.randn((s.B, s.Hkv, s.T, s.dk), generator=g, device="cuda").to(dt)
    v = torch.randn((s.B, s.Hkv, s.T, s.dv), generator=g, device="cuda").to(dt)
    sel, o = nsa.dsa_prefill(s, hi, di, topk, qi, wi, ki, q, k, v)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    Q, K, V = np64(q), np64(k), np64(v)
    QI, WI, KI = np64(qi), np64(wi), np64(ki)
    scale = 1 / math.sqrt(s.dk)
    rng = np.random.default_rng(92)
    rows = sorted({(b, int(t)) for b in range(s.B) for t in
                   list(rng.integers(0, s.T, 12)) + [0, topk - 1, topk, s.T - 1]})
    n_same = 0
    for b, t in rows:
        sc = dsa.index_scores(QI[b, t], WI[b, t], KI[b], t + 1)
        n_same += _check_selection(sc, QI[b, t], WI[b, t], KI[b], t + 1, sel[b, t], topk, (name, b, t))
        ref = dsa.attend(Q[b, t], K[b], V[b], sel[b, t], s.G, scale)   # over the GPU's own (valid) list
        assert np.abs(np64(o[b, t]) - ref).max() <= out_tol(s, ref), (name, b, t)
    assert n_same >= 1
    # injected oracle selection for every position
    ref_all = dsa.dsa_prefill(QI, WI, KI, Q, K, V, topk, s.G, scale)
    sin = np.stack([np.stack([ref_all[(b, t)][0] for t in range(s.T)]) for b in range(s.B)]).astype(np.int32)
    _, o2 = nsa.dsa_prefill(s, hi, di, topk, None, None, None, q, k, v, sel_in=torch.from_numpy(sin).cuda())
    torch.cuda.synchronize()
    O2 = np64(o2)
    for b, t in rows:
        ref = ref_all[(b, t)][1]
        assert np.abs(O2[b, t] - ref).max() <= out_tol(s, ref), ("injected", name, b, t)


@pytest.mark.parametrize("T", [16384, 65536])
def test_dsa_prefill_full_size_sampled(T):
    """4 KV heads x 16, d_k=192, d_v=128, top-2,048 with 4 indexer heads of
    64 at T=16384 (the fwd+bwd workload's shape) and T=65536 (the indexer
    scores held one chunk of rows at a time): 12 positions' selections and
    their attention (the oracle's selection injected at those positions)."""
    s = WORKLOADS["bf16_fwdbwd_T16384"].shape.with_(T=T)
    say("dsa prefill full size", s)
    topk, hi, di = 2048, 4, 64
    g = torch.Generator(device="cuda").manual_seed(93)
    dt = torch.bfloat16
    qi = (torch.randn((s.B, s.T, hi, di), generator=g, device="cuda") / math.sqrt(di)).to(dt)
    wi = (torch.randn((s.B, s.T, hi), generator=g, device="cuda") / math.sqrt(hi)).to(dt)
    ki = torch.randn((s.B, s.T, di), generator=g, device="cuda").to(dt)
    q = torch.randn((s.B, s.T, s.Hq, s.dk), generator=g, device="cuda").to(dt)
    k = torch.randn((s.B, s.Hkv, s.T, s.dk), generator=g, device="cuda").to(dt)
    v = torch.randn((s.B, s.Hkv, s.T, s.dv), generator=g, device="cuda").to(dt)
    ws = nsa.workspace(s, nsa.OP_DSA_PREFILL, "cuda")
    assert ws.numel() <= 256 << 20
    sel, o = nsa.dsa_prefill(s, hi, di, topk, qi, wi, ki, q, k, v, ws=ws)
    torch.cuda.synchronize()
    QI, WI, KI = np64(qi), np64(wi), np64(ki)
    rows = [0, 1, 2047, 2048, 5000, 9999, 12345, T - 1] + list(np.random.default_rng(94).integers(0, s.T, 4))
    sel_np = sel.cpu().numpy()
    sin = sel.clone()
    for t in rows:
        sc = dsa.index_scores(QI[0, t], WI[0, t], KI[0], t + 1)
        _check_selection(sc, QI[0, t], WI[0, t], KI[0], t + 1, sel_np[0, t], topk, ("full", t))
        sin[0, t] = torch.from_numpy(dsa.select_topk(sc, topk).astype(np.int32)).cuda()
    _, o2 = nsa.dsa_prefill(s, hi, di, topk, None, None, None, q, k, v, sel_in=sin)
    torch.cuda.synchronize()
    Kb, Vb = np64(k[0]), np64(v[0])
    for t in rows:
        ref = dsa.attend(np64(q[0, t]), Kb, Vb, sin[0, t].cpu().numpy(), s.G, 1 / math.sqrt(s.dk))
        assert np.abs(np64(o2[0, t]) - ref).max() <= out_tol(s, ref), t
    # rows whose selection was left as the GPU's own: the same bits as the first run
    keep = torch.ones(s.T, dtype=torch.bool, device="cuda")
    keep[torch.tensor(rows, device="cuda")] = False
    assert torch.equal(o2[0, keep], o[0, keep])

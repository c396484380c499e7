"""Block lists given by the caller are sets: order does not matter, a repeated
block counts once, and entries outside 0..floor(t/64) (negative, past the
row's last block, past the sequence) add nothing.  Forward, S4 in one call,
the decode step and the backward take such lists and are compared with the
oracle given the same lists (allinfo.ai.kr DSA explainer, "쉽게 이해하기": the
selected branch normalises over the selected set only)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_attention_long_07_amd import nsa
from sparse_attention_long_07_amd.config import FP32, NSAShape
from sparse_attention_long_07_amd.inputs import make_decode, make_prefill, torch_dtype
from tests.parity_util import grad_tol, np64, ocfg, oracle_compress, out_tol, random_selection

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nsa.lib()


def junk_lists(s: NSAShape, seed: int, t_of=None) -> np.ndarray:
    """random_selection's lists (shuffled, sometimes a repeated entry, -1
    padded) with some padding replaced by blocks past the row's last one,
    by a block far past the sequence and by negative values other than -1.
    t_of(b, t) maps a list to the position it serves (decode: one per
    sequence)."""
    idx = random_selection(s, seed)
    rng = np.random.default_rng(seed + 1000)
    for b, g, t, k in np.argwhere(idx < 0):
        tt = t if t_of is None else t_of(b, t)
        r = rng.random()
        if r < 0.3:
            idx[b, g, t, k] = tt // s.lsel + 1 + int(rng.integers(0, 4))
        elif r < 0.4:
            idx[b, g, t, k] = 1 << 20
        elif r < 0.5:
            idx[b, g, t, k] = -7
    return idx


CASES = [
    ("bf16_T900_g16", NSAShape(1, 900, 2, 16, 192, 128)),
    ("bf16_T700_g16_d64_B2", NSAShape(2, 700, 1, 16, 64, 64, n=5, w=100)),
    ("fp32_T500_g4", NSAShape(1, 500, 1, 4, 64, 64, FP32)),
]


@pytest.mark.parametrize("name,s", CASES, ids=[c[0] for c in CASES])
def test_prefill_lists_are_sets(name, s):
    say("index sets, prefill", name, s)
    x = make_prefill(s, 31, "cuda", unit_scaled=False, with_grad=True)
    dt = torch_dtype(s)
    kc = oracle_compress(s, x["k"], x["w_ck"], x["pe_k"])
    vc = oracle_compress(s, x["v"], x["w_cv"], x["pe_v"])
    idx = junk_lists(s, 32)
    n_junk = int(((idx > np.arange(s.T)[None, None, :, None] // s.lsel) | (idx < -1)).sum())
    say("  entries outside the causal blocks: %d" % n_junk)
    assert n_junk > 0
    ref = orc.forward(ocfg(s), np64(x["q"]), kc, vc, np64(x["k"]), np64(x["v"]), np64(x["w_g"]), np64(x["b_g"]),
                      idx_in=idx)
    kc_d = torch.from_numpy(kc).to(dt).cuda()
    vc_d = torch.from_numpy(vc).to(dt).cuda()
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    o, idx_out = nsa.forward(s, x["q"], x["k"], x["v"], kc_d, vc_d, x["w_g"], x["b_g"], idx_in=idx_d, want_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_out, idx_d)   # the lists used are reported as given
    err = np.abs(np64(o) - ref["o"]).max()
    say("  forward max|o-o_ref| = %.3g (tol %.3g)" % (err, out_tol(s, ref["o"])))
    assert err <= out_tol(s, ref["o"])
    # S4 in one call on the same lists, after S2 on the same compressed keys
    o_cmp, _ = nsa.compressed_attention(s, x["q"], kc_d, vc_d)
    o4 = nsa.sparse_attention(s, x["q"], x["k"], x["v"], o_cmp, idx_d, x["w_g"], x["b_g"])
    torch.cuda.synchronize()
    assert torch.equal(o4, o)
    # backward on the same lists, both forms
    ref_b = orc.backward(ocfg(s), *[np64(x[n]) for n in ("q", "k", "v", "w_ck", "pe_k", "w_cv", "pe_v", "w_g",
                                                          "b_g")], idx, np64(x["do"]), round_bf16=(s.dtype != FP32))
    _, saved = nsa.forward_train(s, x["q"], x["k"], x["v"], kc_d, vc_d, x["w_g"], x["b_g"], idx_in=idx_d)
    for sv in (None, saved):
        g = nsa.backward(s, x["q"], x["k"], x["v"], kc_d, vc_d, x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"],
                         x["w_g"], x["b_g"], idx_d, x["do"], saved=sv)
        torch.cuda.synchronize()
        for rn, gn in (("dq", "d_q"), ("dk", "d_k"), ("dv", "d_v"), ("dwcv", "d_wcv"), ("dwg", "d_wg")):
            e = float(np.abs(np64(g[gn]) - ref_b[rn]).max())
            assert e <= grad_tol(s, ref_b[rn]), (gn, sv is not None, e, grad_tol(s, ref_b[rn]))


def test_decode_lists_are_sets():
    s = NSAShape(4, 1500, 2, 16, 192, 128)
    seq = [1500, 777, 64, 1]
    say("index sets, decode", s, seq)
    x = make_decode(s, 33, "cuda", unit_scaled=False, seq_lens=seq)
    dt = torch_dtype(s)
    kc = oracle_compress(s, x["k"], x["w_ck"], x["pe_k"])
    vc = oracle_compress(s, x["v"], x["w_cv"], x["pe_v"])
    tl = np.array(seq) - 1
    # one list per (sequence, KV head): drawn for a one-position shape per
    # sequence and taken at that position
    lists = np.empty((s.B, s.Hkv, s.n), dtype=np.int32)
    for b in range(s.B):
        sb = s.with_(B=1, T=int(seq[b]))
        lists[b] = junk_lists(sb, 40 + b)[0, :, -1]
    ref = orc.forward_rows(ocfg(s), np.arange(s.B), tl, np64(x["q"]), kc, vc, np64(x["k"]), np64(x["v"]),
                           np64(x["w_g"]), np64(x["b_g"]), idx_in=lists)
    kc_d = torch.from_numpy(kc).to(dt).cuda()
    vc_d = torch.from_numpy(vc).to(dt).cuda()
    idx_d = torch.from_numpy(lists).cuda()
    o = nsa.decode_step(s, x["seq_lens"], x["q"], x["k"], x["v"], kc_d, vc_d, x["w_g"], x["b_g"], idx_in=idx_d)
    torch.cuda.synchronize()
    err = np.abs(np64(o) - ref["o"]).max()
    say("  decode max|o-o_ref| = %.3g (tol %.3g)" % (err, out_tol(s, ref["o"])))
    assert err <= out_tol(s, ref["o"])

"""Long sequences on the matrix-core paths: a 128k prefill (131,072 tokens:
2,048 selection blocks, past the 1,024 blocks the selector's fast path
handles), a decode step on 80,000-token caches and the backward at T=65536,
each compared with the oracle on sampled rows."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_attention_long_07_amd import nsa
from sparse_attention_long_07_amd.config import NSAShape
from sparse_attention_long_07_amd.inputs import make_decode, make_prefill
from tests.parity_util import check_idx, compressed_close, np64, ocfg, oracle_compress, out_tol

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nsa.lib()


def test_prefill_128k_sampled():
    s = NSAShape(1, 131072, 1, 16, 192, 128)
    say("128k prefill", s)
    x = make_prefill(s, 1020, "cuda", unit_scaled=False)
    ck, cv = nsa.compress_kv(s, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"])
    o, idx = nsa.forward(s, x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"], want_idx=True)
    torch.cuda.synchronize()
    kc = oracle_compress(s, x["k"], x["w_ck"], x["pe_k"])
    vc = oracle_compress(s, x["v"], x["w_cv"], x["pe_v"])
    assert compressed_close(s, np64(ck), kc) and compressed_close(s, np64(cv), vc)
    T = s.T
    rows = np.array(sorted(set(range(0, T, 4096)) |
                           {0, 31, 63, 64, 1023, 1024, 65535, 65536, 65599, 65600, 98304, T - 65, T - 64, T - 2, T - 1}),
                    dtype=np.int32)
    rows_t = torch.from_numpy(rows).long().cuda()
    qr = np64(x["q"][0, rows_t])
    k64, v64 = np64(x["k"]), np64(x["v"])
    wg, bg = np64(x["w_g"]), np64(x["b_g"])
    oc = ocfg(s)
    zeros = np.zeros(len(rows), np.int32)
    say("  oracle rows", len(rows))
    ref = orc.forward_rows(oc, zeros, rows, qr, kc, vc, k64, v64, wg, bg, want_scores=True)
    ig = idx.cpu().numpy()[0][:, rows].transpose(1, 0, 2)          # [R, Hkv, n]
    n_exact, n_all = check_idx(s, ref["scores"].reshape(-1, s.nb), np.repeat(rows, s.Hkv),
                               ref["idx"].reshape(-1, s.n), ig.reshape(-1, s.n))
    say("  idx rows checked exactly: %d / %d" % (n_exact, n_all))
    # the oracle's lists injected at the sampled rows
    inj = idx.clone()
    inj[0][:, rows_t] = torch.from_numpy(np.ascontiguousarray(ref["idx"].transpose(1, 0, 2))).cuda()
    o_inj = nsa.forward(s, x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"], idx_in=inj)
    torch.cuda.synchronize()
    tol = out_tol(s, ref["o"])
    err = np.abs(np64(o_inj[0, rows_t]) - ref["o"]).max()
    say("  oracle idx injected: max|o-o_ref| = %.3g (tol %.3g)" % (err, tol))
    assert err <= tol
    # the GPU's own lists, the oracle given the same lists
    ref2 = orc.forward_rows(oc, zeros, rows, qr, kc, vc, k64, v64, wg, bg, idx_in=ig)
    err2 = np.abs(np64(o[0, rows_t]) - ref2["o"]).max()
    say("  own selection: max|o-o_ref| = %.3g" % err2)
    assert err2 <= out_tol(s, ref2["o"])


def test_decode_80k_caches():
    s = NSAShape(2, 80000, 1, 16, 192, 128)
    seq = [80000, 66001]
    say("decode on 80k caches", s, seq)
    x = make_decode(s, 1021, "cuda", unit_scaled=False, seq_lens=seq)
    kc = oracle_compress(s, x["k"], x["w_ck"], x["pe_k"])
    vc = oracle_compress(s, x["v"], x["w_cv"], x["pe_v"])
    kc_d = torch.from_numpy(kc).to(torch.bfloat16).cuda()
    vc_d = torch.from_numpy(vc).to(torch.bfloat16).cuda()
    o, idx = nsa.decode_step(s, x["seq_lens"], x["q"], x["k"], x["v"], kc_d, vc_d, x["w_g"], x["b_g"],
                             want_idx=True)
    torch.cuda.synchronize()
    tl = np.array(seq) - 1
    oc = ocfg(s)
    ref = orc.forward_rows(oc, np.arange(s.B), tl, np64(x["q"]), kc, vc, np64(x["k"]), np64(x["v"]),
                           np64(x["w_g"]), np64(x["b_g"]), want_scores=True)
    n_exact, n_all = check_idx(s, ref["scores"].reshape(-1, s.nb), np.repeat(tl, s.Hkv), ref["idx"].reshape(-1, s.n),
                               idx.cpu().numpy().reshape(-1, s.n))
    say("  idx rows checked exactly: %d / %d" % (n_exact, n_all))
    ref2 = orc.forward_rows(oc, np.arange(s.B), tl, np64(x["q"]), kc, vc, np64(x["k"]), np64(x["v"]),
                            np64(x["w_g"]), np64(x["b_g"]), idx_in=idx.cpu().numpy())
    err = np.abs(np64(o) - ref2["o"]).max()
    say("  max|o-o_ref| = %.3g (tol %.3g)" % (err, out_tol(s, ref2["o"])))
    assert err <= out_tol(s, ref2["o"])
    # the oracle's lists injected
    o3 = nsa.decode_step(s, x["seq_lens"], x["q"], x["k"], x["v"], kc_d, vc_d, x["w_g"], x["b_g"],
                         idx_in=torch.from_numpy(np.ascontiguousarray(ref["idx"]).astype(np.int32)).cuda())
    torch.cuda.synchronize()
    assert np.abs(np64(o3) - ref["o"]).max() <= out_tol(s, ref["o"])


def test_backward_64k_masked_do():
    """The backward at T=65536 (one KV group of 16 heads, d_k=192, d_v=128),
    both forms, against the oracle's exact gradients for a dO that is zero
    outside 32 sampled rows and the last 192 (so the oracle visits only those
    rows); d_q must be zero on every other row."""
    from tests.parity_util import random_selection
    from tests.test_gpu_backward import PAIRS, _gpu_bwd, _gpu_saved, _oracle_bwd, _tol

    s = NSAShape(1, 65536, 1, 16, 192, 128)
    say("64k backward", s)
    x = make_prefill(s, 14, "cuda", unit_scaled=False, with_grad=True)
    ck, cv = nsa.compress_kv(s, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"])
    x["cmp_k"], x["cmp_v"] = ck, cv
    x["idx"] = torch.from_numpy(random_selection(s, 13)).cuda()
    T = s.T
    t0 = T - 192
    rng = np.random.default_rng(15)
    rows = np.unique(np.concatenate([rng.choice(t0, size=24, replace=False), [0, 31, 63, 64, 511, 512, 32767, 32768]]))
    keep = np.zeros(T, dtype=bool)
    keep[rows] = True
    keep[t0:] = True
    do_mask = x["do"].clone()
    do_mask[:, torch.from_numpy(~keep).cuda()] = 0
    say("  oracle backward on", int(keep.sum()), "rows")
    ref = _oracle_bwd(s, x, np64(do_mask))
    for saved in (None, _gpu_saved(s, x)):
        g = _gpu_bwd(s, x, do_mask, saved)
        for rn, gn in PAIRS:
            err = float(np.abs(np64(g[gn]) - ref[rn]).max())
            say("  ", gn, "saved" if saved is not None else "recomputed", "max err %.3g tol %.3g" % (err, _tol(s, ref, rn)))
            assert err <= _tol(s, ref, rn), (gn, saved is not None, err)
        assert not np.any(np64(g["d_q"])[:, ~keep])

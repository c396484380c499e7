"""Parity of the HIP backward pass (nsa_backward, through the C ABI) with the
oracle's backward on the same seeded inputs and the same fixed selection.

Small cases: every gradient element by element.  The 16k bf16 fwd+bwd
workload: the oracle gives exact gradients for a dO that is zero outside a
set of rows, so the GPU runs twice -- with the full N(0,1) dO (dq on the
kept rows and dk/dv on the last keys, which only the kept tail rows reach,
are compared) and with the masked dO (every gradient tensor is compared)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_attention_long_07_amd import nsa
from sparse_attention_long_07_amd.config import BF16, FP32, WORKLOADS, NSAShape
from sparse_attention_long_07_amd.inputs import make_prefill, torch_dtype
from tests.parity_util import grad_tol, np64, ocfg, oracle_compress, random_selection

pytestmark = pytest.mark.gpu

PAIRS = (("dq", "d_q"), ("dk", "d_k"), ("dv", "d_v"), ("dwck", "d_wck"), ("dpek", "d_pek"), ("dwcv", "d_wcv"),
         ("dpev", "d_pev"), ("dwg", "d_wg"), ("dbg", "d_bg"))
NAMES = ("q", "k", "v", "w_ck", "pe_k", "w_cv", "pe_v", "w_g", "b_g")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nsa.lib()


def _setup(s, seed, scaled, idx=None):
    """Inputs on the GPU, the oracle's compressed K/V (exact in the storage
    dtype) on both sides, and the selection: the oracle's own when idx is
    None."""
    x = make_prefill(s, seed, "cuda", unit_scaled=scaled, with_grad=True)
    dt = torch_dtype(s)
    kc = oracle_compress(s, x["k"], x["w_ck"], x["pe_k"])
    vc = oracle_compress(s, x["v"], x["w_cv"], x["pe_v"])
    if idx is None:
        idx = orc.forward(ocfg(s), np64(x["q"]), kc, vc, np64(x["k"]), np64(x["v"]), np64(x["w_g"]),
                          np64(x["b_g"]))["idx"]
    x["cmp_k"] = torch.from_numpy(kc).to(dt).cuda()
    x["cmp_v"] = torch.from_numpy(vc).to(dt).cuda()
    x["idx"] = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    return x


def _gpu_bwd(s, x, d_o, saved=None):
    g = nsa.backward(s, x["q"], x["k"], x["v"], x["cmp_k"], x["cmp_v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"],
                     x["w_g"], x["b_g"], x["idx"], d_o, saved=saved)
    torch.cuda.synchronize()
    return g


def _gpu_saved(s, x):
    """The training forward's saved statistics for x's inputs and selection."""
    _, saved = nsa.forward_train(s, x["q"], x["k"], x["v"], x["cmp_k"], x["cmp_v"], x["w_g"], x["b_g"],
                                 idx_in=x["idx"])
    torch.cuda.synchronize()
    return saved


# Gradients that cancel to (near) zero in exact arithmetic take the scale of a
# counterpart that does not: dPE_k always (a common shift of every compressed
# key), dK when a row's softmax has a single key (then ds = p (dP - D) = 0), and
# dW_k when every row sees at most one compressed key (T < 47: the compressed
# keys' gradient is then zero, and so is its weight gradient).
COMPANION = {"dpek": "dpev", "dk": "dv", "dwck": "dwcv"}


def _tol(s, ref, rn):
    c = COMPANION.get(rn)
    own = float(np.abs(ref[rn]).max())
    if c and own < 1e-3 * float(np.abs(ref[c]).max()):
        return grad_tol(s, ref[rn], float(np.abs(ref[c]).max()))
    return grad_tol(s, ref[rn])


def _oracle_bwd(s, x, d_o_np):
    return orc.backward(ocfg(s), *[np64(x[n]) for n in NAMES], x["idx"].cpu().numpy(), d_o_np,
                        round_bf16=(s.dtype == BF16))


SMALL = [
    ("fp32_T1024", NSAShape(1, 1024, 1, 4, 64, 64, FP32), True, False),
    ("bf16_T777_g16", NSAShape(1, 777, 2, 16, 192, 128), False, False),
    ("bf16_T1000_n6_w128_randsel", NSAShape(1, 1000, 1, 16, 192, 128, n=6, w=128), False, True),
    ("bf16_odd_dims_B2", NSAShape(2, 333, 3, 3, 24, 40, n=5, w=100), False, True),
    ("fp32_T300_g5_w64", NSAShape(1, 300, 2, 5, 32, 16, FP32, n=3, w=64), False, False),
    ("bf16_T31", NSAShape(1, 31, 1, 2, 16, 16), False, False),
    ("fp32_T1", NSAShape(1, 1, 1, 1, 8, 8, FP32), True, False),
    # matrix-core raw-key pass at the other head widths, over 2 and 3 row chunks
    ("bf16_T1500_g16_d64_B2H2_randsel", NSAShape(2, 1500, 2, 16, 64, 64, n=6, w=200), False, True),
    ("bf16_T2100_g16_d128_randsel", NSAShape(1, 2100, 1, 16, 128, 128, n=8, w=256), False, True),
    # K/V of a key chunk too wide to stage in LDS: read in place
    ("fp32_T260_g16_d256_unstaged", NSAShape(1, 260, 1, 16, 256, 256, FP32, n=4, w=100), False, True),
    # matrix-core passes with a window shorter than a selection block (selected blocks shared with the
    # window sweep and window rows carrying both branches start mid-block), and with the window
    # covering the whole sequence
    ("bf16_T700_g16_d64_w40_randsel", NSAShape(1, 700, 1, 16, 64, 64, n=5, w=40), False, True),
    ("bf16_T600_g16_d128_wT_randsel", NSAShape(1, 600, 2, 16, 128, 128, n=4, w=1024), False, True),
    # matrix-core passes with no compressed block (T < 32) and with one (T = 47)
    ("bf16_T20_g16", NSAShape(1, 20, 1, 16, 192, 128), False, False),
    ("bf16_T300_g16_d64_Hkv3_randsel", NSAShape(1, 300, 3, 16, 64, 64, n=4, w=100), False, True),
    ("bf16_T47_g16_d64_B2_randsel", NSAShape(2, 47, 1, 16, 64, 64, n=4, w=40), False, True),
]


@pytest.mark.parametrize("name,s,scaled,randsel", SMALL, ids=[c[0] for c in SMALL])
def test_backward_parity(name, s, scaled, randsel):
    """Both forms of the call: recomputing every branch's statistics, and
    with the training forward's saved statistics."""
    say("backward", name, s)
    x = _setup(s, 5, scaled, random_selection(s, 6) if randsel else None)
    ref = _oracle_bwd(s, x, np64(x["do"]))
    for saved in (None, _gpu_saved(s, x)):
        g = _gpu_bwd(s, x, x["do"], saved)
        for rn, gn in PAIRS:
            got = np64(g[gn])
            assert got.shape == ref[rn].shape, gn
            err = float(np.abs(got - ref[rn]).max())
            assert err <= _tol(s, ref, rn), (gn, saved is not None, err, _tol(s, ref, rn))


def test_backward_deterministic():
    s = NSAShape(1, 700, 2, 16, 192, 128)
    say("backward determinism", s)
    x = _setup(s, 7, False, random_selection(s, 8))
    g1 = _gpu_bwd(s, x, x["do"])
    g2 = _gpu_bwd(s, x, x["do"])
    for _, gn in PAIRS:
        assert torch.equal(g1[gn], g2[gn]), gn
    saved = _gpu_saved(s, x)
    g1 = _gpu_bwd(s, x, x["do"], saved)
    g2 = _gpu_bwd(s, x, x["do"], saved)
    for _, gn in PAIRS:
        assert torch.equal(g1[gn], g2[gn]), gn


def test_backward_full_size():
    """bf16, T=16384, 4 KV groups x 16 heads, d_k=192, d_v=128, the launch
    configuration of the fwd+bwd workload; N(0,1) inputs and dO."""
    w = WORKLOADS["bf16_fwdbwd_T16384"]
    s = w.shape
    say("backward full size", s)
    sel = random_selection(s, 11)
    x = make_prefill(s, 10, "cuda", unit_scaled=w.unit_scaled, with_grad=True)
    dt = torch_dtype(s)
    # the GPU's own compression is used on both sides here (the oracle
    # recomputes it in fp64; rounding differences stay far inside the bound)
    ck, cv = nsa.compress_kv(s, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"])
    x["cmp_k"], x["cmp_v"] = ck, cv
    x["idx"] = torch.from_numpy(sel).cuda()
    T = s.T
    t0 = T - 192
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([rng.choice(t0, size=24, replace=False), [0, 31, 63, 64, 511, 512]]))
    keep = np.zeros(T, dtype=bool)
    keep[rows] = True
    keep[t0:] = True
    do_full = x["do"]
    do_mask = do_full.clone()
    do_mask[:, torch.from_numpy(~keep).cuda()] = 0
    say("oracle backward on", int(keep.sum()), "rows")
    ref = _oracle_bwd(s, x, np64(do_mask))
    say("gpu backward, masked dO")
    g = _gpu_bwd(s, x, do_mask.to(dt))
    for rn, gn in PAIRS:
        got = np64(g[gn])
        err = float(np.abs(got - ref[rn]).max())
        say(gn, "max err", err, "tol", _tol(s, ref, rn))
        assert err <= _tol(s, ref, rn), (gn, err)
    assert not np.any(np64(g["d_q"])[:, ~keep])
    say("gpu backward, masked dO, saved statistics")
    g = _gpu_bwd(s, x, do_mask.to(dt), _gpu_saved(s, x))
    for rn, gn in PAIRS:
        got = np64(g[gn])
        err = float(np.abs(got - ref[rn]).max())
        say(gn, "max err", err, "tol", _tol(s, ref, rn))
        assert err <= _tol(s, ref, rn), (gn, err)
    assert not np.any(np64(g["d_q"])[:, ~keep])
    say("gpu backward, full dO")
    g = _gpu_bwd(s, x, do_full)
    dq = np64(g["d_q"])[:, keep]
    assert float(np.abs(dq - ref["dq"][:, keep]).max()) <= grad_tol(s, ref["dq"][:, keep])
    for rn, gn in (("dk", "d_k"), ("dv", "d_v")):
        got = np64(g[gn])[:, :, t0:]
        r = ref[rn][:, :, t0:]
        assert float(np.abs(got - r).max()) <= grad_tol(s, r), gn

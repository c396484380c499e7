"""Parity of the HIP backward pass with the two-layer compression map
(nsa_backward_mlp, through the C ABI) with the oracle's backward_mlp, on the
same seeded inputs and the same fixed selection: every gradient element by
element, both layers' weight gradients included."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_attention_long_07_amd import nsa
from sparse_attention_long_07_amd.config import BF16, FP32, NSAShape
from sparse_attention_long_07_amd.inputs import make_mlp_weights, make_prefill, torch_dtype
from tests.parity_util import grad_tol, np64, ocfg, random_selection

pytestmark = pytest.mark.gpu

PAIRS = (("dq", "d_q"), ("dk", "d_k"), ("dv", "d_v"), ("dw1k", "d_w1k"), ("dpek", "d_pek"), ("dw2k", "d_w2k"),
         ("dw1v", "d_w1v"), ("dpev", "d_pev"), ("dw2v", "d_w2v"), ("dwg", "d_wg"), ("dbg", "d_bg"))
# gradients that cancel to (near) zero take the scale of a counterpart
COMPANION = {"dpek": "dpev", "dk": "dv"}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nsa.lib()


def _tol(s, ref, rn):
    c = COMPANION.get(rn)
    own = float(np.abs(ref[rn]).max())
    if c and own < 1e-3 * float(np.abs(ref[c]).max()):
        return grad_tol(s, ref[rn], float(np.abs(ref[c]).max()))
    return grad_tol(s, ref[rn])


CASES = [
    ("fp32_T1024", NSAShape(1, 1024, 1, 4, 64, 64, FP32), True, False),
    ("bf16_T777_g16", NSAShape(1, 777, 2, 16, 192, 128), False, False),
    ("bf16_odd_dims_B2_randsel", NSAShape(2, 333, 3, 3, 24, 40, n=5, w=100), False, True),
    ("bf16_T2100_g16_d128_randsel", NSAShape(1, 2100, 1, 16, 128, 128, n=8, w=256), False, True),
    ("fp32_T300_g5_w64", NSAShape(1, 300, 2, 5, 32, 16, FP32, n=3, w=64), False, False),
    ("bf16_T31", NSAShape(1, 31, 1, 2, 16, 16), False, False),
    ("bf16_T20_g16", NSAShape(1, 20, 1, 16, 192, 128), False, False),
]


@pytest.mark.parametrize("name,s,scaled,randsel", CASES, ids=[c[0] for c in CASES])
def test_backward_mlp_parity(name, s, scaled, randsel):
    say("backward mlp", name, s)
    rb = s.dtype == BF16
    dt = torch_dtype(s)
    x = make_prefill(s, 21, "cuda", unit_scaled=scaled, with_grad=True)
    w = make_mlp_weights(s, 22, "cuda")
    # the oracle's compressed K/V (exact in the storage dtype) on both sides
    kc = orc.compress_mlp(np64(x["k"]), np64(x["w_ck"]), np64(x["pe_k"]), np64(w["w2_k"]), s.l, s.d, s.n_pad,
                          round_bf16=rb)
    vc = orc.compress_mlp(np64(x["v"]), np64(x["w_cv"]), np64(x["pe_v"]), np64(w["w2_v"]), s.l, s.d, s.n_pad,
                          round_bf16=rb)
    if randsel:
        idx = random_selection(s, 23)
    else:
        idx = orc.forward(ocfg(s), np64(x["q"]), kc, vc, np64(x["k"]), np64(x["v"]), np64(x["w_g"]),
                          np64(x["b_g"]))["idx"]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    kc_d, vc_d, idx_d = torch.from_numpy(kc).to(dt).cuda(), torch.from_numpy(vc).to(dt).cuda(), torch.from_numpy(idx).cuda()
    ref = orc.backward_mlp(ocfg(s), np64(x["q"]), np64(x["k"]), np64(x["v"]), np64(x["w_ck"]), np64(x["pe_k"]),
                           np64(w["w2_k"]), np64(x["w_cv"]), np64(x["pe_v"]), np64(w["w2_v"]), np64(x["w_g"]),
                           np64(x["b_g"]), idx, np64(x["do"]), round_bf16=rb)
    # recomputed statistics, then the training forward's saved ones
    _, saved = nsa.forward_train(s, x["q"], x["k"], x["v"], kc_d, vc_d, x["w_g"], x["b_g"], idx_in=idx_d)
    for sv in (None, saved):
        g = nsa.backward_mlp(s, x["q"], x["k"], x["v"], kc_d, vc_d, x["w_ck"], x["pe_k"], w["w2_k"], x["w_cv"],
                             x["pe_v"], w["w2_v"], x["w_g"], x["b_g"], idx_d, x["do"], saved=sv)
        torch.cuda.synchronize()
        for rn, gn in PAIRS:
            got = np64(g[gn])
            assert got.shape == ref[rn].shape, gn
            err = float(np.abs(got - ref[rn]).max())
            assert np.all(np.isfinite(got)), gn
            assert err <= _tol(s, ref, rn), (gn, sv is not None, err, _tol(s, ref, rn))


def test_backward_mlp_deterministic():
    s = NSAShape(1, 700, 2, 16, 192, 128)
    say("backward mlp determinism", s)
    x = make_prefill(s, 24, "cuda", unit_scaled=False, with_grad=True)
    w = make_mlp_weights(s, 25, "cuda")
    ck, cv = nsa.compress_kv_mlp(s, x["k"], x["v"], x["w_ck"], x["pe_k"], w["w2_k"], x["w_cv"], x["pe_v"], w["w2_v"])
    idx = torch.from_numpy(random_selection(s, 26)).cuda()
    args = (s, x["q"], x["k"], x["v"], ck, cv, x["w_ck"], x["pe_k"], w["w2_k"], x["w_cv"], x["pe_v"], w["w2_v"],
            x["w_g"], x["b_g"], idx, x["do"])
    g1 = nsa.backward_mlp(*args)
    g2 = nsa.backward_mlp(*args)
    torch.cuda.synchronize()
    for _, gn in PAIRS:
        assert torch.equal(g1[gn], g2[gn]), gn

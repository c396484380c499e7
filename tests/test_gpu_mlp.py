"""Two-layer compression map (nsa_compress_kv_mlp) against the oracle.

Tolerance, from the arithmetic: both sides round the hidden layer
a = W1 vec(block + PE) and the output W2 relu(a) to the storage type.  The
GPU accumulates in fp32, so a hidden value near a rounding boundary may round
one unit (2^-7 relative in bf16) the other way; each output c can then move
by at most 2^-7 sum_j |W2[c][j]| |h_j|, plus one unit of its own rounding.
Such flips are rare: outside the bound without them, at most 2% of entries
may differ.  With W2 = I and nonnegative pre-activations the network is the
linear map, so the GPU result must equal nsa_compress_kv bit for bit."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import oracle as orc
from sparse_attention_long_07_amd import nsa
from sparse_attention_long_07_amd.config import BF16, FP32, WORKLOADS, NSAShape
from sparse_attention_long_07_amd.inputs import make_mlp_weights, make_prefill
from tests.parity_util import np64

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nsa.lib()


def _oracle(s, x, W1, PE, W2, n_out):
    rb = s.dtype == BF16
    out = orc.compress_mlp(np64(x), np64(W1), np64(PE), np64(W2), s.l, s.d, n_out, round_bf16=rb)
    hid = np.maximum(orc.compress(np64(x), np64(W1), np64(PE), s.l, s.d, n_out, round_bf16=rb), 0.0)
    return out, hid


def _check(s, got, ref, hid, W2, where):
    W2 = np.abs(np64(W2))
    prop = hid @ W2.T                          # sum_j |W2[c][j]| |h_j|
    dim = ref.shape[-1]
    if s.dtype == BF16:
        unit = 2.0 ** -7
        base = unit * np.abs(ref) + 2.0 ** -16 * prop
        bound = base + unit * prop
    else:
        unit = 2.0 ** -20
        floor = 64 * np.sqrt(32 * dim) * 2.0 ** -24 * max(float(np.abs(hid).max()), 1e-30)
        base = unit * np.abs(ref) + unit * prop + floor * W2.sum(axis=1)
        bound = base
    err = np.abs(got - ref)
    assert np.all(err <= bound), (where, float(err.max()), float((err - bound).max()))
    assert float(np.mean(err > base)) <= 0.02, (where, float(np.mean(err > base)))


CASES = [
    # matrix-core second layer (d = 192 / 128, 64)
    ("bf16_T1100_d192", NSAShape(1, 1100, 2, 16, 192, 128)),
    ("bf16_T700_d64_B2", NSAShape(2, 700, 1, 16, 64, 64, n=5, w=200)),
    ("bf16_T47_d128", NSAShape(1, 47, 1, 16, 128, 128)),
    # vector-ALU second layer: other widths, fp32
    ("bf16_odd_B2", NSAShape(2, 400, 3, 3, 24, 40, n=5, w=100)),
    ("fp32_T600", NSAShape(2, 600, 1, 4, 64, 64, FP32)),
    # no complete block: every row is a pad
    ("bf16_T31", NSAShape(1, 31, 1, 2, 16, 16)),
]


@pytest.mark.parametrize("name,s", CASES, ids=[c[0] for c in CASES])
def test_mlp_compression_parity(name, s):
    say("mlp compression", name, s)
    x = make_prefill(s, 71, "cuda")
    w = make_mlp_weights(s, 72, "cuda")
    ck, cv = nsa.compress_kv_mlp(s, x["k"], x["v"], x["w_ck"], x["pe_k"], w["w2_k"], x["w_cv"], x["pe_v"],
                                 w["w2_v"])
    torch.cuda.synchronize()
    for got, xx, W1, PE, W2, tag in ((ck, x["k"], x["w_ck"], x["pe_k"], w["w2_k"], "K"),
                                     (cv, x["v"], x["w_cv"], x["pe_v"], w["w2_v"], "V")):
        ref, hid = _oracle(s, xx, W1, PE, W2, s.n_pad)
        g = np64(got)
        _check(s, g, ref, hid, W2, (name, tag))
        assert np.all(g[:, :, s.n_cmp:] == 0.0), (name, tag)


@pytest.mark.parametrize("name,s", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_mlp_identity_equals_linear_map(name, s):
    """W2 = I and every pre-activation >= 0: bit for bit the linear map."""
    say("mlp identity", name, s)
    x = make_prefill(s, 73, "cuda")
    for key in ("k", "v", "w_ck", "pe_k", "w_cv", "pe_v"):
        x[key] = x[key].abs()
    dt = x["k"].dtype
    ik = torch.eye(s.dk, dtype=dt, device="cuda")
    iv = torch.eye(s.dv, dtype=dt, device="cuda")
    lk, lv = nsa.compress_kv(s, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"])
    mk, mv = nsa.compress_kv_mlp(s, x["k"], x["v"], x["w_ck"], x["pe_k"], ik, x["w_cv"], x["pe_v"], iv)
    torch.cuda.synchronize()
    assert torch.equal(mk, lk) and torch.equal(mv, lv)


def test_mlp_compression_full_size_sampled():
    """bf16 T=65536, 4 KV heads, d_k=192, d_v=128 (the prefill workload's
    shape): 40 sampled blocks per KV head against the oracle on their own
    32 tokens, and the pads."""
    s = WORKLOADS["bf16_T65536"].shape
    say("mlp compression full size", s)
    x = make_prefill(s, 74, "cuda")
    w = make_mlp_weights(s, 75, "cuda")
    ck, cv = nsa.compress_kv_mlp(s, x["k"], x["v"], x["w_ck"], x["pe_k"], w["w2_k"], x["w_cv"], x["pe_v"],
                                 w["w2_v"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(76)
    blocks = np.unique(np.concatenate([[0, 1, s.n_cmp - 1], rng.integers(0, s.n_cmp, 37)]))
    one = NSAShape(1, 32, 1, s.G, s.dk, s.dv, s.dtype)
    for got, xx, W1, PE, W2, tag in ((ck, x["k"], x["w_ck"], x["pe_k"], w["w2_k"], "K"),
                                     (cv, x["v"], x["w_cv"], x["pe_v"], w["w2_v"], "V")):
        for h in range(s.Hkv):
            sl = torch.stack([xx[0, h, 16 * int(i):16 * int(i) + 32] for i in blocks])[:, None]   # [n,1,32,dim]
            ref, hid = _oracle(one, sl, W1, PE, W2, 1)
            g = np64(got[0, h, blocks])[:, None, None, :]
            _check(s, g, ref, hid, W2, ("full", tag, h))
        assert bool((got[:, :, s.n_cmp:] == 0).all())

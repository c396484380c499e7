"""Pins of the oracle's backward pass (reverse mode through compression, the
three branches and the gates, with the block selection held fixed).

The gradients are checked against central finite differences of the oracle's
forward pass, which is itself pinned elsewhere against library attention,
closed forms and the pages' numbers.  Every input tensor gets its own random
direction u; (L(x + eps u) - L(x - eps u)) / (2 eps) must equal <grad, u>.
A dropped term, a wrong sign, a wrong token index or a transposed weight in
the backward changes <grad, u> by far more than the tolerance.  CPU only."""
import math

import numpy as np
import pytest

from oracle import oracle as orc

NAMES = ("q", "k", "v", "wck", "pek", "wcv", "pev", "wg", "bg")
GRADS = ("dq", "dk", "dv", "dwck", "dpek", "dwcv", "dpev", "dwg", "dbg")


def make(T, B=1, Hkv=2, G=2, dk=16, dv=8, n=4, w=48, seed=0):
    rng = np.random.default_rng(seed)
    cfg = orc.Cfg(B, T, Hkv, G, dk, dv, n=n, w=w)
    Hq = Hkv * G
    x = dict(
        q=rng.standard_normal((B, T, Hq, dk)),
        k=rng.standard_normal((B, Hkv, T, dk)),
        v=rng.standard_normal((B, Hkv, T, dv)),
        wck=rng.standard_normal((dk, 32 * dk)) / math.sqrt(32 * dk),
        pek=rng.standard_normal((32, dk)) / math.sqrt(dk),
        wcv=rng.standard_normal((dv, 32 * dv)) / math.sqrt(32 * dv),
        pev=rng.standard_normal((32, dv)) / math.sqrt(dv),
        wg=rng.standard_normal((Hq, 3, dk)) / math.sqrt(dk),
        bg=rng.standard_normal((Hq, 3)) / math.sqrt(dk),
    )
    # a fixed selection: the always-kept blocks plus random others, in random
    # order, with a repeated entry now and then (the branch uses the set)
    idx = -np.ones((B, Hkv, T, n), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            for t in range(T):
                jc = t // 64
                s = sorted({0, max(jc - 1, 0), jc})
                rest = [j for j in range(jc + 1) if j not in s]
                rng.shuffle(rest)
                s = s + rest[: n - len(s)]
                if len(s) < n and rng.random() < 0.5:
                    s.append(s[0])
                rng.shuffle(s)
                idx[b, g, t, : len(s)] = s
    dO = rng.standard_normal((B, T, Hq, dv))
    return cfg, x, idx, dO


def loss(cfg, x, idx, dO):
    npad = max(64, -(-orc.n_cmp(cfg.T) // 64) * 64)
    kc = orc.compress(x["k"], x["wck"], x["pek"], n_out=npad)
    vc = orc.compress(x["v"], x["wcv"], x["pev"], n_out=npad)
    o = orc.forward(cfg, x["q"], kc, vc, x["k"], x["v"], x["wg"], x["bg"], idx_in=idx)["o"]
    return float(np.sum(o * dO))


def grads(cfg, x, idx, dO):
    return orc.backward(cfg, *[x[nm] for nm in NAMES], idx, dO)


CASES = {
    # ragged last selection block, several compression blocks, window < block
    "T250_w48_n4": dict(T=250, w=48, n=4),
    # two sequences, window wider than a block, every block selectable
    "T200_B2_w100_n16": dict(T=200, B=2, w=100, n=16),
    # the finite-difference size, pages' window and count
    "T256_w512_n16": dict(T=256, w=512, n=16, G=3, dk=8, dv=16),
}


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_finite_differences(case):
    cfg, x, idx, dO = make(**CASES[case])
    gr = grads(cfg, x, idx, dO)
    rng = np.random.default_rng(99)
    eps = 1e-5
    # rounding noise of the difference quotient: ~|L| * 1e-15 / eps
    floor = 1e-9 * (1.0 + abs(loss(cfg, x, idx, dO)))
    for nm, gn in zip(NAMES, GRADS):
        u = rng.standard_normal(x[nm].shape)
        xp = dict(x)
        xm = dict(x)
        xp[nm] = x[nm] + eps * u
        xm[nm] = x[nm] - eps * u
        fd = (loss(cfg, xp, idx, dO) - loss(cfg, xm, idx, dO)) / (2 * eps)
        an = float(np.sum(gr[gn] * u))
        scale = float(np.sum(np.abs(gr[gn] * u))) + 1e-12
        assert abs(fd - an) <= 1e-7 * scale + floor, (nm, fd, an)


def test_backward_single_elements():
    """Element-wise finite differences at places with a special role: the
    first token (in every branch's first block), a token that two compression
    blocks share, the last token of a ragged sequence, a position embedding
    slot, and the gate bias of each branch."""
    cfg, x, idx, dO = make(T=250, w=48, n=4)
    gr = grads(cfg, x, idx, dO)
    eps = 1e-5
    picks = [("k", "dk", (0, 0, 0, 3)), ("k", "dk", (0, 1, 40, 5)), ("v", "dv", (0, 1, 40, 2)),
             ("k", "dk", (0, 0, 249, 0)), ("v", "dv", (0, 0, 249, 7)), ("q", "dq", (0, 0, 1, 4)),
             ("q", "dq", (0, 249, 3, 0)), ("pek", "dpek", (17, 2)), ("pev", "dpev", (31, 1)),
             ("wck", "dwck", (5, 16 * 20 + 3)), ("wcv", "dwcv", (7, 8 * 31 + 7)),
             ("bg", "dbg", (1, 0)), ("bg", "dbg", (2, 1)), ("bg", "dbg", (3, 2))]
    for nm, gn, ix in picks:
        xp = dict(x)
        xm = dict(x)
        xp[nm] = x[nm].copy()
        xm[nm] = x[nm].copy()
        xp[nm][ix] += eps
        xm[nm][ix] -= eps
        fd = (loss(cfg, xp, idx, dO) - loss(cfg, xm, idx, dO)) / (2 * eps)
        assert abs(fd - gr[gn][ix]) <= 1e-7 * (abs(fd) + 1.0), (nm, ix, fd, gr[gn][ix])


def test_compressed_key_shift_invariance():
    """PE_k adds the same vector W_ck vec(PE_k) to every compressed key, which
    shifts all logits of a row by one constant; the softmax ignores that, so
    dPE_k = 0 and the compressed-key gradients of each (sequence, KV head)
    sum to zero.  dPE_v is not zero: PE_v shifts o_cmp itself."""
    cfg, x, idx, dO = make(T=250, w=48, n=4)
    gr = grads(cfg, x, idx, dO)
    ref = np.abs(gr["dwck"]).max()
    assert np.abs(gr["dpek"]).max() <= 1e-12 * ref
    assert np.abs(gr["dpev"]).max() > 1e-3
    # dW_ck is then independent of PE_k
    x2 = dict(x)
    x2["pek"] = x["pek"] + 3.0
    gr2 = grads(cfg, x2, idx, dO)
    assert np.allclose(gr2["dwck"], gr["dwck"], rtol=0, atol=1e-12 * ref)


def test_backward_no_compressed_block():
    """T < 32: no compression block exists, so o_cmp = 0 on every row; the
    compression weights and the compressed gate get exactly zero gradient,
    while the other two gates do not."""
    cfg, x, idx, dO = make(T=31, w=512, n=16)
    gr = grads(cfg, x, idx, dO)
    for gn in ("dwck", "dpek", "dwcv", "dpev"):
        assert not np.any(gr[gn])
    assert not np.any(gr["dbg"][:, 0]) and not np.any(gr["dwg"][:, 0])
    assert np.all(gr["dbg"][:, 1:] != 0)


# ---------------------------------------------------------------------------
# The two-layer compression map (compress_mlp): first layer w1 with the
# position encoding, ReLU, second layer w2.

MLP_NAMES = ("q", "k", "v", "w1k", "pek", "w2k", "w1v", "pev", "w2v", "wg", "bg")
MLP_GRADS = ("dq", "dk", "dv", "dw1k", "dpek", "dw2k", "dw1v", "dpev", "dw2v", "dwg", "dbg")


def make_mlp(T, seed=1, **kw):
    cfg, x, idx, dO = make(T, seed=seed, **kw)
    rng = np.random.default_rng(seed + 100)
    dk, dv = cfg.dk, cfg.dv
    x = dict(x)
    x["w1k"] = x.pop("wck")
    x["w1v"] = x.pop("wcv")
    x["w2k"] = rng.standard_normal((dk, dk)) / math.sqrt(dk)
    x["w2v"] = rng.standard_normal((dv, dv)) / math.sqrt(dv)
    return cfg, x, idx, dO


def loss_mlp(cfg, x, idx, dO):
    npad = max(64, -(-orc.n_cmp(cfg.T) // 64) * 64)
    kc = orc.compress_mlp(x["k"], x["w1k"], x["pek"], x["w2k"], n_out=npad)
    vc = orc.compress_mlp(x["v"], x["w1v"], x["pev"], x["w2v"], n_out=npad)
    o = orc.forward(cfg, x["q"], kc, vc, x["k"], x["v"], x["wg"], x["bg"], idx_in=idx)["o"]
    return float(np.sum(o * dO))


def grads_mlp(cfg, x, idx, dO):
    return orc.backward_mlp(cfg, *[x[nm] for nm in MLP_NAMES], idx, dO)


@pytest.mark.parametrize("case", ["T250_w48_n4", "T200_B2_w100_n16"])
def test_backward_mlp_matches_finite_differences(case):
    """Every input of the two-layer map's backward against central
    differences of the oracle's forward (compress_mlp feeding forward).  The
    ReLU's kink is crossed by no difference quotient here: the smallest
    |hidden value| of these inputs is far above eps times its directional
    derivative."""
    cfg, x, idx, dO = make_mlp(**CASES[case])
    gr = grads_mlp(cfg, x, idx, dO)
    rng = np.random.default_rng(98)
    eps = 1e-5
    floor = 1e-9 * (1.0 + abs(loss_mlp(cfg, x, idx, dO)))
    for nm, gn in zip(MLP_NAMES, MLP_GRADS):
        u = rng.standard_normal(x[nm].shape)
        xp = dict(x)
        xm = dict(x)
        xp[nm] = x[nm] + eps * u
        xm[nm] = x[nm] - eps * u
        fd = (loss_mlp(cfg, xp, idx, dO) - loss_mlp(cfg, xm, idx, dO)) / (2 * eps)
        an = float(np.sum(gr[gn] * u))
        scale = float(np.sum(np.abs(gr[gn] * u))) + 1e-12
        assert abs(fd - an) <= 1e-7 * scale + floor, (nm, fd, an)


def test_backward_mlp_single_elements():
    """Element-wise differences in both layers' weights, a position encoding
    slot and a token two compression blocks share."""
    cfg, x, idx, dO = make_mlp(T=250, w=48, n=4)
    gr = grads_mlp(cfg, x, idx, dO)
    eps = 1e-5
    picks = [("w2k", "dw2k", (3, 11)), ("w2v", "dw2v", (7, 0)), ("w1k", "dw1k", (5, 16 * 20 + 3)),
             ("w1v", "dw1v", (2, 8 * 31 + 7)), ("pev", "dpev", (31, 1)), ("k", "dk", (0, 1, 40, 5)),
             ("v", "dv", (0, 0, 249, 7))]
    for nm, gn, ix in picks:
        xp = dict(x)
        xm = dict(x)
        xp[nm] = x[nm].copy()
        xm[nm] = x[nm].copy()
        xp[nm][ix] += eps
        xm[nm][ix] -= eps
        fd = (loss_mlp(cfg, xp, idx, dO) - loss_mlp(cfg, xm, idx, dO)) / (2 * eps)
        assert abs(fd - gr[gn][ix]) <= 1e-7 * (abs(fd) + 1.0), (nm, ix, fd, gr[gn][ix])


def test_backward_mlp_reduces_to_linear():
    """With w2 = I and every hidden value positive (non-negative tokens, first
    layer weights and position encodings), the two-layer map is the linear
    map with w1: every gradient the linear backward reports is the same.  The
    second layer's gradient is dw2 = sum_i dC_i a_i^T with a_i = w1 X_i, while
    the linear backward gives dwc = sum_i dC_i X_i^T, so dw2 = dwc w1^T."""
    cfg, x, idx, dO = make_mlp(T=200, B=2, w=100, n=16, seed=3)
    for nm in ("k", "v", "w1k", "w1v", "pek", "pev"):
        x[nm] = np.abs(x[nm])
    x["w2k"] = np.eye(cfg.dk)
    x["w2v"] = np.eye(cfg.dv)
    gm = grads_mlp(cfg, x, idx, dO)
    gl = orc.backward(cfg, x["q"], x["k"], x["v"], x["w1k"], x["pek"], x["w1v"], x["pev"], x["wg"], x["bg"], idx, dO)
    for a, b in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("dw1k", "dwck"), ("dpek", "dpek"),
                 ("dw1v", "dwcv"), ("dpev", "dpev"), ("dwg", "dwg"), ("dbg", "dbg")):
        # dpek is zero up to rounding (PE_k shifts every compressed key alike),
        # so the scale is the weight gradient's for it
        ref = max(np.abs(gl[b]).max(), np.abs(gl["dwck"]).max() * (b == "dpek"))
        assert np.abs(gm[a] - gl[b]).max() <= 1e-12 * ref, a
    # a = w1 X for each row, so sum_i dC_i a_i^T = (sum_i dC_i X_i^T) w1^T = dwc w1^T
    for a, b, w in (("dw2k", "dwck", "w1k"), ("dw2v", "dwcv", "w1v")):
        ref = gl[b] @ x[w].T
        assert np.abs(gm[a] - ref).max() <= 1e-10 * (np.abs(ref).max() + 1e-30), a


def test_backward_mlp_dead_hidden_layer():
    """Every hidden value negative (non-negative tokens and position encodings,
    non-positive first layer): the compressed keys and values are all zero, so
    neither layer nor the position encodings get a gradient, and the raw-key,
    query and gate gradients equal those of a linear map whose weights are
    zero."""
    cfg, x, idx, dO = make_mlp(T=250, w=48, n=4, seed=4)
    for nm in ("k", "v", "pek", "pev"):
        x[nm] = np.abs(x[nm])
    for nm in ("w1k", "w1v"):
        x[nm] = -np.abs(x[nm]) - 1e-3
    gm = grads_mlp(cfg, x, idx, dO)
    for nm in ("dw1k", "dpek", "dw2k", "dw1v", "dpev", "dw2v"):
        assert np.all(gm[nm] == 0.0), nm
    z = {nm: np.zeros_like(x[nm]) for nm in ("w1k", "w1v")}
    gl = orc.backward(cfg, x["q"], x["k"], x["v"], z["w1k"], x["pek"], z["w1v"], x["pev"], x["wg"], x["bg"], idx, dO)
    for nm in ("dq", "dk", "dv", "dwg", "dbg"):
        assert np.abs(gm[nm] - gl[nm]).max() <= 1e-12 * (np.abs(gl[nm]).max() + 1e-30), nm

"""The C ABI without a GPU: the library loads, exports every function that
include/nsa.h declares, sizes workspaces, and rejects bad arguments on the
host before anything reaches HIP.  Fake device pointers are never
dereferenced because every call here fails its host-side checks."""
import ctypes
import os
import re

import pytest

from sparse_attention_long_07_amd import nsa
from sparse_attention_long_07_amd.config import WORKLOADS, NSAShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "nsa.h")

NULL, SHAPE, DTYPE, PARAM, WS, HIP, ALIGN = -1, -2, -3, -4, -5, -6, -7
FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced
MIS = ctypes.c_void_p(0x10004)         # misaligned


def declared_functions():
    text = open(HDR).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(nsa_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    L = nsa.lib()
    decl = declared_functions()
    assert set(decl) == set(nsa.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings():
    L = nsa.lib()
    for code in [0, NULL, SHAPE, DTYPE, PARAM, WS, HIP, ALIGN]:
        assert L.nsa_status_string(code).decode() != "unknown status"
    assert L.nsa_status_string(12345).decode() == "unknown status"


def cfg(**kw):
    s = NSAShape(1, 256, 2, 4, 64, 32, "bf16")
    c = nsa.config(s)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_workspace_bytes():
    for w in WORKLOADS.values():
        s = w.shape
        f = nsa.workspace_bytes(s, nsa.OP_FORWARD)
        d = nsa.workspace_bytes(s, nsa.OP_DECODE)
        assert f >= s.esize * s.B * s.T * s.Hq * s.dv    # compressed-branch output
        assert d >= s.esize * s.B * s.Hq * s.dv
        assert f % 256 == 0 and d % 256 == 0
    L = nsa.lib()
    assert L.nsa_workspace_bytes(ctypes.byref(cfg(T=0)), 0) == 0
    assert L.nsa_workspace_bytes(ctypes.byref(cfg()), 99) == 0
    assert L.nsa_workspace_bytes(None, 0) == 0


BAD_CONFIGS = [
    (dict(dtype=2), DTYPE),
    (dict(B=0), SHAPE), (dict(T=0), SHAPE), (dict(T=524289), SHAPE), (dict(H_kv=0), SHAPE),
    (dict(group=0), SHAPE), (dict(group=17), SHAPE), (dict(d_k=12), SHAPE), (dict(d_k=264), SHAPE),
    (dict(d_v=0), SHAPE),
    (dict(l=16), PARAM), (dict(d=8), PARAM), (dict(l_sel=32), PARAM), (dict(n=2), PARAM), (dict(n=17), PARAM),
    (dict(w=0), PARAM), (dict(w=8193), PARAM), (dict(scale=-1.0), PARAM), (dict(scale=float("nan")), PARAM),
]


@pytest.mark.parametrize("kw,code", BAD_CONFIGS)
def test_bad_config_rejected_everywhere(kw, code):
    L = nsa.lib()
    c = ctypes.byref(cfg(**kw))
    f = [FAKE] * 16
    assert L.nsa_compress_kv(c, *f[:8], None) == code
    assert L.nsa_compress_kv_mlp(c, *f[:10], None) == code
    assert L.nsa_compress_append(c, f[0], f[1], 1, *f[:8], None) == code
    assert L.nsa_compress_append_mlp(c, f[0], f[1], 1, *f[:10], None) == code
    assert L.nsa_select_blocks(c, f[0], f[1], None, f[2], f[3], 1 << 40, None) == code
    assert L.nsa_forward(c, *f[:7], None, f[0], None, None, f[1], 1 << 40, None) == code
    assert L.nsa_forward_train(c, *f[:7], None, f[0], None, None, f[1], f[2], f[3], 1 << 40, None) == code
    assert L.nsa_decode_step(c, *f[:8], None, f[0], None, f[1], 1 << 40, None) == code
    assert L.nsa_backward(c, *([FAKE] * 22), None, None, FAKE, 1 << 40, None) == code
    assert L.nsa_backward_mlp(c, *([FAKE] * 26), None, None, FAKE, 1 << 40, None) == code
    assert L.nsa_dsa_decode(c, 4, 64, 16, *([FAKE] * 10), FAKE, 1 << 40, None) == code
    assert L.nsa_dsa_prefill(c, 4, 64, 16, *([FAKE] * 9), FAKE, 1 << 40, None) == code
    assert L.nsa_sparse_attention(c, *f[:8], f[0], 1 << 40, None) == code
    assert L.nsa_window_attention(c, *f[:7], None) == code
    assert L.nsa_pack_kv_blocks(c, f[0], f[1], f[2], 1 << 40, None) == code
    assert L.nsa_selected_attention(c, *f[:7], f[0], 1 << 40, None) == code
    assert L.nsa_compressed_attention(c, *f[:5], None) == code
    assert L.nsa_compressed_window_attention(c, *f[:10], f[0], 1 << 40, None) == code
    assert L.nsa_select_topn(c, f[0], f[1], None) == code


def test_null_config():
    L = nsa.lib()
    assert L.nsa_compress_kv(None, *[FAKE] * 8, None) == NULL
    assert L.nsa_forward(None, *[FAKE] * 12, 1 << 40, None) == NULL


@pytest.mark.parametrize("pos", range(8))
def test_compress_null_and_misaligned(pos):
    L = nsa.lib()
    c = ctypes.byref(cfg())
    args = [FAKE] * 8
    args[pos] = None
    assert L.nsa_compress_kv(c, *args, None) == NULL
    args[pos] = MIS
    assert L.nsa_compress_kv(c, *args, None) == ALIGN


@pytest.mark.parametrize("pos", range(10))
def test_compress_mlp_null_and_misaligned(pos):
    """k v w1_k pe_k w2_k w1_v pe_v w2_v cmp_k cmp_v: all required, 16-byte aligned."""
    L = nsa.lib()
    c = ctypes.byref(cfg())
    args = [FAKE] * 10
    args[pos] = None
    assert L.nsa_compress_kv_mlp(c, *args, None) == NULL
    args[pos] = MIS
    assert L.nsa_compress_kv_mlp(c, *args, None) == ALIGN


@pytest.mark.parametrize("pos", range(9))
def test_compress_append_checks(pos):
    """len_new and the eight tensors are required (len_old may be NULL); every
    failing call returns before anything is enqueued."""
    L = nsa.lib()
    c = ctypes.byref(cfg())
    args = [FAKE] * 9           # len_new | k_cache v_cache w_ck pe_k w_cv pe_v cmp_k cmp_v
    args[pos] = None
    assert L.nsa_compress_append(c, None, args[0], 16, *args[1:], None) == NULL
    if pos > 0:
        args[pos] = MIS
        assert L.nsa_compress_append(c, FAKE, args[0], 16, *args[1:], None) == ALIGN
    # max_append must lie in 1..T (T = 256 here)
    f = [FAKE] * 8
    for bad in (0, -1, 257):
        assert L.nsa_compress_append(c, FAKE, FAKE, bad, *f, None) == PARAM


@pytest.mark.parametrize("pos", range(11))
def test_compress_append_mlp_checks(pos):
    """As test_compress_append_checks, with both layers' weights."""
    L = nsa.lib()
    c = ctypes.byref(cfg())
    args = [FAKE] * 11          # len_new | k_cache v_cache w1_k pe_k w2_k w1_v pe_v w2_v cmp_k cmp_v
    args[pos] = None
    assert L.nsa_compress_append_mlp(c, None, args[0], 16, *args[1:], None) == NULL
    if pos > 0:
        args[pos] = MIS
        assert L.nsa_compress_append_mlp(c, FAKE, args[0], 16, *args[1:], None) == ALIGN
    f = [FAKE] * 10
    for bad in (0, -1, 257):
        assert L.nsa_compress_append_mlp(c, FAKE, FAKE, bad, *f, None) == PARAM


@pytest.mark.parametrize("pos", range(8))
def test_forward_required_pointers(pos):
    L = nsa.lib()
    c = ctypes.byref(cfg())
    args = [FAKE] * 8           # q k v cmp_k cmp_v w_g b_g | o
    args[pos] = None
    q, k, v, ck, cv, wg, bg, o = args
    assert L.nsa_forward(c, q, k, v, ck, cv, wg, bg, None, o, None, None, FAKE, 1 << 40, None) == NULL


def test_forward_workspace_checks():
    L = nsa.lib()
    c = cfg()
    need = L.nsa_workspace_bytes(ctypes.byref(c), 0)
    f = [FAKE] * 7
    assert L.nsa_forward(ctypes.byref(c), *f, None, FAKE, None, None, None, need, None) == WS
    assert L.nsa_forward(ctypes.byref(c), *f, None, FAKE, None, None, FAKE, need - 1, None) == WS
    assert L.nsa_forward(ctypes.byref(c), *f, None, FAKE, None, None, ctypes.c_void_p(0x10010), need,
                         None) == ALIGN
    # optional outputs are checked for alignment too
    assert L.nsa_forward(ctypes.byref(c), *f, MIS, FAKE, None, None, FAKE, 0, None) == ALIGN


@pytest.mark.parametrize("pos", range(10))
def test_forward_train_checks(pos):
    """nsa_forward_train: the forward's operands plus lse and o_branch, all
    required and 16-byte aligned; workspace as nsa_forward's."""
    L = nsa.lib()
    c = cfg()
    need = L.nsa_workspace_bytes(ctypes.byref(c), nsa.OP_FORWARD)
    args = [FAKE] * 10          # q k v cmp_k cmp_v w_g b_g | o | lse o_branch
    args[pos] = None
    q, k, v, ck, cv, wg, bg, o, lse, obr = args
    assert L.nsa_forward_train(ctypes.byref(c), q, k, v, ck, cv, wg, bg, None, o, None, None, lse, obr, FAKE, need,
                               None) == NULL
    args[pos] = MIS
    q, k, v, ck, cv, wg, bg, o, lse, obr = args
    assert L.nsa_forward_train(ctypes.byref(c), q, k, v, ck, cv, wg, bg, None, o, None, None, lse, obr, FAKE, need,
                               None) == ALIGN
    f = [FAKE] * 7
    assert L.nsa_forward_train(ctypes.byref(c), *f, None, FAKE, None, None, FAKE, FAKE, FAKE, need - 1, None) == WS


@pytest.mark.parametrize("mlp", [False, True])
def test_backward_saved_pair_checks(mlp):
    """The saved statistics go in pairs (lse with o_branch) and are aligned."""
    L = nsa.lib()
    c = ctypes.byref(cfg())
    fn, nreq, op = (L.nsa_backward_mlp, 26, nsa.OP_BACKWARD_MLP) if mlp else (L.nsa_backward, 22, nsa.OP_BACKWARD)
    need = L.nsa_workspace_bytes(c, op)
    args = [FAKE] * nreq
    assert fn(c, *args, FAKE, None, FAKE, need, None) == NULL
    assert fn(c, *args, None, FAKE, FAKE, need, None) == NULL
    assert fn(c, *args, MIS, FAKE, FAKE, need, None) == ALIGN
    assert fn(c, *args, FAKE, MIS, FAKE, need, None) == ALIGN
    assert fn(c, *args, FAKE, FAKE, FAKE, need - 1, None) == WS


def test_select_and_decode_checks():
    L = nsa.lib()
    c = cfg()
    assert L.nsa_select_blocks(ctypes.byref(c), FAKE, FAKE, None, None, FAKE, 1 << 40, None) == NULL
    assert L.nsa_select_blocks(ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, 0, None) == WS
    need = L.nsa_workspace_bytes(ctypes.byref(c), 2)
    f = [FAKE] * 7
    assert L.nsa_decode_step(ctypes.byref(c), None, *f, None, FAKE, None, FAKE, need, None) == NULL
    assert L.nsa_decode_step(ctypes.byref(c), FAKE, *f, None, FAKE, None, FAKE, need - 256, None) == WS


def test_dsa_decode_checks():
    """Shapes the matrix-core attention takes, indexer sizes, required
    pointers (the indexer's only without sel_in), alignment, workspace."""
    L = nsa.lib()
    ok = cfg(group=16, d_k=192, d_v=128, dtype=1)
    c = ctypes.byref(ok)
    f = [FAKE] * 7     # q_idx w_idx k_idx q k v | sel_in
    need = L.nsa_workspace_bytes(c, 5)
    assert need >= 4 * ok.B * ok.T
    # unsupported attention shapes
    for bad in (cfg(group=16, d_k=192, d_v=128, dtype=0), cfg(group=8, d_k=192, d_v=128, dtype=1),
                cfg(group=16, d_k=96, d_v=96, dtype=1)):
        assert L.nsa_dsa_decode(ctypes.byref(bad), 4, 64, 2048, FAKE, *f[:6], None, FAKE, FAKE, FAKE, need,
                                None) == SHAPE
    # indexer sizes and k
    for hi, di, k in ((0, 64, 16), (17, 64, 16), (4, 4, 16), (4, 260, 16), (4, 60, 16), (4, 64, 0), (4, 64, 8193)):
        assert L.nsa_dsa_decode(c, hi, di, k, FAKE, *f[:6], None, FAKE, FAKE, FAKE, need, None) == PARAM
    # required pointers
    assert L.nsa_dsa_decode(c, 4, 64, 16, None, *f[:6], None, FAKE, FAKE, FAKE, need, None) == NULL
    for pos in range(6):
        a = list(f[:6])
        a[pos] = None
        assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, *a, None, FAKE, FAKE, FAKE, need, None) == NULL
    assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, *f[:6], None, None, FAKE, FAKE, need, None) == NULL   # sel_out
    assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, *f[:6], None, FAKE, None, FAKE, need, None) == NULL   # o
    # with sel_in the indexer's inputs, sel_out and ws may be NULL; misalignment still caught
    assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, None, None, None, MIS, FAKE, FAKE, FAKE, None, FAKE, None, 0,
                            None) == ALIGN
    assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, MIS, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need,
                            None) == ALIGN
    # workspace
    assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, *f[:6], None, FAKE, FAKE, None, need, None) == WS
    assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, *f[:6], None, FAKE, FAKE, FAKE, need - 256, None) == WS
    # the reported size always holds the two-way split's partials (per (b, g, half): 16 maxima,
    # 16 sums, 16 x d_v outputs in fp32), so the selection and the split run together
    assert need >= 4 * ok.B * ok.H_kv * 2 * (32 + 16 * ok.d_v) and need % 256 == 0
    # a workspace not 256-byte aligned is rejected, with or without sel_in
    W16 = ctypes.c_void_p(0x10010)
    assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, *f[:6], None, FAKE, FAKE, W16, need, None) == ALIGN
    assert L.nsa_dsa_decode(c, 4, 64, 16, FAKE, None, None, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, W16, need,
                            None) == ALIGN


def test_dsa_prefill_checks():
    L = nsa.lib()
    ok = cfg(group=16, d_k=128, d_v=128, dtype=1)
    c = ctypes.byref(ok)
    need = L.nsa_workspace_bytes(c, 6)
    assert need >= 4 * ok.B * ok.T * ok.T
    f = [FAKE] * 6     # q_idx w_idx k_idx q k v
    assert L.nsa_dsa_prefill(ctypes.byref(cfg(group=4, d_k=128, d_v=128, dtype=1)), 4, 64, 16, *f, None, FAKE, FAKE,
                             FAKE, need, None) == SHAPE
    assert L.nsa_dsa_prefill(c, 4, 64, 0, *f, None, FAKE, FAKE, FAKE, need, None) == PARAM
    assert L.nsa_dsa_prefill(c, 4, 64, 16, *f, None, None, FAKE, FAKE, need, None) == NULL
    assert L.nsa_dsa_prefill(c, 4, 64, 16, *f, None, FAKE, FAKE, FAKE, need - 256, None) == WS
    assert L.nsa_dsa_prefill(c, 4, 64, 16, FAKE, FAKE, FAKE, MIS, FAKE, FAKE, None, FAKE, FAKE, FAKE, need,
                             None) == ALIGN
    assert L.nsa_dsa_prefill(c, 4, 64, 16, *f, None, FAKE, FAKE, ctypes.c_void_p(0x10010), need, None) == ALIGN
    # the indexer scores are held one chunk of rows at a time: bounded at any length
    big = ctypes.byref(cfg(B=2, T=524288, group=16, d_k=192, d_v=128, dtype=1))
    nb = L.nsa_workspace_bytes(big, 6)
    assert 4 * 524288 <= nb <= 256 << 20 and nb % 256 == 0
    mid = ctypes.byref(cfg(B=1, T=65536, group=16, d_k=192, d_v=128, dtype=1))
    assert L.nsa_workspace_bytes(mid, 6) == 256 << 20


def test_binding_rejects_host_tensors():
    import torch
    s = NSAShape(1, 64, 1, 2, 16, 16, "fp32")
    t = torch.zeros(1)
    with pytest.raises(ValueError):
        nsa.compress_kv(s, t, t, t, t, t, t)


def test_binding_arity_matches_header():
    """Each ctypes prototype has as many parameters as the header declares."""
    text = open(HDR).read()
    L = nsa.lib()
    for name in declared_functions():
        m = re.search(r"\b%s\s*\(([^)]*)\)" % name, text, re.S)
        nparams = len([p for p in m.group(1).split(",") if p.strip()])
        assert len(getattr(L, name).argtypes) == nparams, name


@pytest.mark.parametrize("pos", range(22))
def test_backward_required_pointers(pos):
    L = nsa.lib()
    c = ctypes.byref(cfg())
    need = L.nsa_workspace_bytes(c, nsa.OP_BACKWARD)
    args = [FAKE] * 22
    args[pos] = None
    assert L.nsa_backward(c, *args, None, None, FAKE, need, None) == NULL
    args[pos] = MIS
    assert L.nsa_backward(c, *args, None, None, FAKE, need, None) == ALIGN


@pytest.mark.parametrize("pos", range(26))
def test_backward_mlp_required_pointers(pos):
    L = nsa.lib()
    c = ctypes.byref(cfg())
    need = L.nsa_workspace_bytes(c, nsa.OP_BACKWARD_MLP)
    args = [FAKE] * 26
    args[pos] = None
    assert L.nsa_backward_mlp(c, *args, None, None, FAKE, need, None) == NULL
    args[pos] = MIS
    assert L.nsa_backward_mlp(c, *args, None, None, FAKE, need, None) == ALIGN


def test_backward_mlp_workspace_checks():
    L = nsa.lib()
    c = cfg()
    need = L.nsa_workspace_bytes(ctypes.byref(c), nsa.OP_BACKWARD_MLP)
    base = L.nsa_workspace_bytes(ctypes.byref(c), nsa.OP_BACKWARD)
    s = NSAShape(1, 256, 2, 4, 64, 32, "bf16")
    # the linear map's workspace plus the hidden layers (bf16) and their gradient (fp32)
    assert need >= base + s.B * s.Hkv * s.n_pad * (2 * (s.dk + s.dv) + 4 * (s.dk + s.dv))
    assert need % 256 == 0
    f = [FAKE] * 26
    assert L.nsa_backward_mlp(ctypes.byref(c), *f, None, None, None, need, None) == WS
    assert L.nsa_backward_mlp(ctypes.byref(c), *f, None, None, FAKE, need - 1, None) == WS
    assert L.nsa_backward_mlp(ctypes.byref(c), *f, None, None, ctypes.c_void_p(0x10010), need, None) == ALIGN
    assert L.nsa_backward_mlp(ctypes.byref(cfg(B=70000, H_kv=1, group=1)), *f, None, None, FAKE, 1 << 40, None) == SHAPE


def test_backward_workspace_checks():
    L = nsa.lib()
    c = cfg()
    need = L.nsa_workspace_bytes(ctypes.byref(c), nsa.OP_BACKWARD)
    s = NSAShape(1, 256, 2, 4, 64, 32, "bf16")
    # per-row statistics, raw-key gradients and compressed-key gradients at least
    assert need >= 4 * (s.B * s.T * s.Hq * 12 + s.B * s.Hkv * s.T * (s.dk + s.dv))
    assert need % 256 == 0
    f = [FAKE] * 22
    assert L.nsa_backward(ctypes.byref(c), *f, None, None, None, need, None) == WS
    assert L.nsa_backward(ctypes.byref(c), *f, None, None, FAKE, need - 1, None) == WS
    assert L.nsa_backward(ctypes.byref(c), *f, None, None, ctypes.c_void_p(0x10010), need, None) == ALIGN
    # B * H_kv above the grid limit of the key passes
    assert L.nsa_backward(ctypes.byref(cfg(B=70000, H_kv=1, group=1)), *f, None, None, FAKE, 1 << 40, None) == SHAPE


@pytest.mark.parametrize("pos", range(8))
def test_sparse_stage_required_pointers(pos):
    """S4 and its two halves reject null and misaligned operands."""
    L = nsa.lib()
    c = ctypes.byref(cfg())
    args = [FAKE] * 8           # q k v o_cmp idx w_g b_g o
    args[pos] = None
    assert L.nsa_sparse_attention(c, *args, FAKE, 1 << 40, None) == NULL
    args[pos] = MIS
    assert L.nsa_sparse_attention(c, *args, FAKE, 1 << 40, None) == ALIGN
    win = [FAKE] * 7            # q k v o_cmp w_g b_g o
    sel = [FAKE] * 7            # q k v idx w_g b_g o
    if pos < 7:
        win[pos] = None
        sel[pos] = None
        assert L.nsa_window_attention(c, *win, None) == NULL
        assert L.nsa_selected_attention(c, *sel, FAKE, 1 << 40, None) == NULL
        win[pos] = MIS
        sel[pos] = MIS
        assert L.nsa_window_attention(c, *win, None) == ALIGN
        assert L.nsa_selected_attention(c, *sel, FAKE, 1 << 40, None) == ALIGN


def test_selected_attention_workspace_checks():
    L = nsa.lib()
    c = nsa.config(NSAShape(1, 256, 2, 16, 128, 128, "bf16"))      # a shape with packed K/V blocks
    need = L.nsa_workspace_bytes(ctypes.byref(c), nsa.OP_SPARSE)
    assert need > 0
    f = [FAKE] * 7
    assert L.nsa_selected_attention(ctypes.byref(c), *f, None, need, None) == WS
    assert L.nsa_selected_attention(ctypes.byref(c), *f, FAKE, need - 1, None) == WS
    assert L.nsa_selected_attention(ctypes.byref(c), *f, ctypes.c_void_p(0x10010), need, None) == ALIGN
    assert L.nsa_sparse_attention(ctypes.byref(c), *([FAKE] * 8), FAKE, need - 1, None) == WS
    assert L.nsa_pack_kv_blocks(ctypes.byref(c), FAKE, FAKE, FAKE, need - 1, None) == WS
    assert L.nsa_pack_kv_blocks(ctypes.byref(c), FAKE, FAKE, None, need, None) == WS
    assert L.nsa_pack_kv_blocks(ctypes.byref(c), None, FAKE, FAKE, need, None) == NULL
    assert L.nsa_pack_kv_blocks(ctypes.byref(c), FAKE, MIS, FAKE, need, None) == ALIGN
    # a shape that reads K and V directly needs no workspace: nothing to pack, no launch
    c2 = nsa.config(NSAShape(1, 256, 2, 4, 64, 32, "bf16"))
    assert L.nsa_workspace_bytes(ctypes.byref(c2), nsa.OP_SPARSE) == 0
    assert L.nsa_pack_kv_blocks(ctypes.byref(c2), FAKE, FAKE, None, 0, None) == 0


@pytest.mark.parametrize("pos", range(3))
def test_compressed_attention_checks(pos):
    """q, cmp_k and scores are required; cmp_v and o_cmp are both given or both
    NULL (scores only); every pointer 16-byte aligned."""
    L = nsa.lib()
    c = ctypes.byref(cfg())
    req = [FAKE] * 3            # q cmp_k scores
    req[pos] = None
    q, ck, sc = req
    assert L.nsa_compressed_attention(c, q, ck, FAKE, FAKE, sc, None) == NULL
    assert L.nsa_compressed_attention(c, q, ck, None, None, sc, None) == NULL
    req[pos] = MIS
    q, ck, sc = req
    assert L.nsa_compressed_attention(c, q, ck, FAKE, FAKE, sc, None) == ALIGN
    # one of cmp_v / o_cmp without the other
    assert L.nsa_compressed_attention(c, FAKE, FAKE, FAKE, None, FAKE, None) == NULL
    assert L.nsa_compressed_attention(c, FAKE, FAKE, None, FAKE, FAKE, None) == NULL
    assert L.nsa_compressed_attention(c, FAKE, FAKE, MIS, FAKE, FAKE, None) == ALIGN
    assert L.nsa_compressed_attention(c, FAKE, FAKE, FAKE, MIS, FAKE, None) == ALIGN


@pytest.mark.parametrize("pos", range(9))
def test_compressed_window_attention_checks(pos):
    """q k v cmp_k cmp_v w_g b_g scores o are required, o_cmp is optional,
    every pointer 16-byte aligned; without o_cmp, a configuration that is
    not one kernel needs a 256-byte aligned workspace for it."""
    L = nsa.lib()
    c = ctypes.byref(cfg())
    req = [FAKE] * 9
    req[pos] = None
    assert L.nsa_compressed_window_attention(c, *req, FAKE, None, 0, None) == NULL
    req[pos] = MIS
    assert L.nsa_compressed_window_attention(c, *req, FAKE, None, 0, None) == ALIGN
    assert L.nsa_compressed_window_attention(c, *([FAKE] * 9), MIS, None, 0, None) == ALIGN
    need = L.nsa_workspace_bytes(c, nsa.OP_CMP_WINDOW)
    s = NSAShape(1, 256, 2, 4, 64, 32, "bf16")
    assert need == (s.esize * s.B * s.T * s.Hq * s.dv + 255) // 256 * 256
    assert L.nsa_compressed_window_attention(c, *([FAKE] * 9), None, None, 0, None) == WS
    assert L.nsa_compressed_window_attention(c, *([FAKE] * 9), None, FAKE, need - 1, None) == WS
    assert L.nsa_compressed_window_attention(c, *([FAKE] * 9), None, ctypes.c_void_p(0x10010), need, None) == ALIGN
    # one kernel (16 heads per KV head, bf16, d_k/d_v = 192/128): no workspace
    one = nsa.config(NSAShape(1, 256, 2, 16, 192, 128, "bf16"))
    assert L.nsa_workspace_bytes(ctypes.byref(one), nsa.OP_CMP_WINDOW) == 0


def test_select_topn_checks():
    L = nsa.lib()
    c = ctypes.byref(cfg())
    assert L.nsa_select_topn(c, None, FAKE, None) == NULL
    assert L.nsa_select_topn(c, FAKE, None, None) == NULL
    assert L.nsa_select_topn(c, MIS, FAKE, None) == ALIGN
    assert L.nsa_select_topn(c, FAKE, MIS, None) == ALIGN
    assert L.nsa_select_topn(None, FAKE, FAKE, None) == NULL


def test_decode_noalloc_checks():
    """The allocation-free decode step checks its arguments before any HIP
    call: bad configurations, NULL and misaligned pointers, and a workspace
    need above its 32 MiB scratch array."""
    L = nsa.lib()
    c = ctypes.byref(cfg())
    f = [FAKE] * 8          # seq_lens q k_cache v_cache cmp_k cmp_v w_g b_g
    assert L.nsa_decode_step_noalloc(ctypes.byref(cfg(T=0)), *f, None, FAKE, None, None) == SHAPE
    assert L.nsa_decode_step_noalloc(None, *f, None, FAKE, None, None) == NULL
    for pos in range(8):
        a = list(f)
        a[pos] = None
        assert L.nsa_decode_step_noalloc(c, *a, None, FAKE, None, None) == NULL
        a[pos] = MIS
        assert L.nsa_decode_step_noalloc(c, *a, None, FAKE, None, None) == ALIGN
    assert L.nsa_decode_step_noalloc(c, *f, None, None, None, None) == NULL          # o
    assert L.nsa_decode_step_noalloc(c, *f, MIS, FAKE, None, None) == ALIGN          # idx_in
    assert L.nsa_decode_step_noalloc(c, *f, None, FAKE, MIS, None) == ALIGN          # idx_out
    # 4,096 sequences of 65,536 tokens need far more than the 32 MiB array
    big = nsa.config(NSAShape(4096, 65536, 4, 16, 192, 128))
    assert L.nsa_workspace_bytes(ctypes.byref(big), nsa.OP_DECODE) > 32 << 20
    assert L.nsa_decode_step_noalloc(ctypes.byref(big), *f, None, FAKE, None, None) == WS
    # the decode workload (32 x 65,536) fits
    wl = nsa.config(WORKLOADS["bf16_decode_B32_T65536"].shape)
    assert 0 < L.nsa_workspace_bytes(ctypes.byref(wl), nsa.OP_DECODE) <= 32 << 20

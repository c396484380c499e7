"""nsa_decode_step_noalloc (the decode step on the library's static scratch
array) against nsa_decode_step (the same step on a caller-owned workspace):
two calls in a row, the second on a smaller input, each equal bit for bit to
the workspace entry point on the same inputs -- the scratch keeps the first
call's contents, which the second must not depend on."""
from __future__ import annotations

import sys

import pytest
import torch

from sparse_attention_long_07_amd import nsa
from sparse_attention_long_07_amd.config import NSAShape
from sparse_attention_long_07_amd.inputs import make_decode

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nsa.lib()


CALLS = [
    # (shape, sequence lengths, seed): the second call is smaller than the first
    (NSAShape(32, 65536, 4, 16, 192, 128), None, 301),
    (NSAShape(3, 5000, 2, 16, 192, 128), [5000, 4097, 77], 302),
]


def _run(s, lens, seed, with_idx_in):
    x = make_decode(s, seed, "cuda", unit_scaled=False, seq_lens=lens)
    ck, cv = nsa.compress_kv(s, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"])
    o_ws, idx_ws = nsa.decode_step(s, x["seq_lens"], x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"], want_idx=True)
    o_na, idx_na = nsa.decode_step_noalloc(s, x["seq_lens"], x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"],
                                           want_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_na, idx_ws)
    assert torch.equal(o_na, o_ws)
    if with_idx_in:
        # the selection injected: the step skips selecting, the rest is the same
        o2 = nsa.decode_step_noalloc(s, x["seq_lens"], x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"],
                                     idx_in=idx_ws)
        torch.cuda.synchronize()
        o3 = nsa.decode_step(s, x["seq_lens"], x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"], idx_in=idx_ws)
        torch.cuda.synchronize()
        assert torch.equal(o2, o3)


def test_noalloc_decode_matches_workspace_decode_twice():
    for i, (s, lens, seed) in enumerate(CALLS):
        say("noalloc decode call", i, s, lens)
        _run(s, lens, seed, with_idx_in=(i == 1))


def test_noalloc_rejects_oversized_workload():
    s = NSAShape(4096, 65536, 4, 16, 192, 128)
    say("noalloc oversized", s)
    assert nsa.workspace_bytes(s, nsa.OP_DECODE) > 32 << 20
    t = torch.zeros(16, dtype=torch.int32, device="cuda")
    import ctypes
    c = nsa.config(s)
    st = nsa.lib().nsa_decode_step_noalloc(ctypes.byref(c), *([ctypes.c_void_p(t.data_ptr())] * 8), None,
                                           ctypes.c_void_p(t.data_ptr()), None, None)
    assert st == -5   # NSA_ERR_WORKSPACE, nothing launched

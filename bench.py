"""NSA benchmark on one MI355X.

One step = the whole hot path over one batch of synthetic input:
  * the 64k prefill forward (B=1, T=65536, 4 KV heads x 16 query heads,
    d_k=192, d_v=128, bf16) as nsa_forward launches it after compression
    (S1): compressed attention with block importance (S2) together with the
    window half of S4 in one kernel, top-n selection (S3), then packing of
    the K/V blocks and the selected half of S4 with the gated sum;
  * one decode step on 32 sequences with 65,536-token caches (same heads).
Inputs are resident in HBM before timing starts.  Each stage is bracketed by
HIP events on the stream the kernels run on; the printed JSON line carries
the prefill throughput (the headline metric), the decode step time, the
roofline of the dominant kernel and the CPU oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import math
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_attention_long_07_amd import nsa  # noqa: E402
from sparse_attention_long_07_amd.config import (WORKLOADS, backward_flops, decode_bytes, decode_flops,  # noqa: E402
                                                 decode_slots, prefill_flops)
from sparse_attention_long_07_amd.inputs import (make_decode, make_dsa_indexer, make_mlp_weights,  # noqa: E402
                                                 make_prefill)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0

# HBM bytes per launch of a kernel from the FETCH_SIZE and WRITE_SIZE counters
# (scaled by a plain device copy's readings), with the source file(s) they were
# taken on and their SHA-256: the figure is reported only while those sources
# are unchanged.
MEASURED_TRAFFIC = {
    "k_selected_mfma": ("sparse_attention_long_07_amd/csrc/k_sparse.hip",
                        "44a66c0b754df24b5e81780b0588c8a12a37842d851c7b1c6c85a64f2de53085", 63.16e9),
    "k_cmp_attn_mfma+window": ([("sparse_attention_long_07_amd/csrc/k_cmp_attn.hip",
                                 "87cd1dd624260d4ecdf2552ed97c4deab85161ecc3a576b3a349e344a069f7f8"),
                                ("sparse_attention_long_07_amd/csrc/window_phase.h",
                                 "c6c0db9e68159d260edbf8d4d9ec3cbe63465c2724d7ddfa440db8ff653f1bb4")], 4.416e9),
}


def measured_traffic(kernel):
    """HBM bytes per launch from the committed counter summary, while the
    kernel's sources (one path or several, each with its SHA-256) are the
    ones it was measured on; else None."""
    ent = MEASURED_TRAFFIC.get(kernel)
    if ent is None:
        return None
    *srcs, nbytes = ent
    pairs = [srcs] if isinstance(srcs[0], str) else srcs[0]
    for path, sha in pairs:
        with open(os.path.join(ROOT, path), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != sha:
                return None
    return nbytes


def dsa_decode(s, y, steps, topk=2048, hi=4, di=64):
    """The DSA-style decode step (indexer, top-k tokens, attention over them)
    on the decode workload's caches, timed apart from the headline step."""
    dev = y["k"].device
    ix = make_dsa_indexer(s, 1006, dev, hi, di)
    sel = torch.empty((s.B, topk), dtype=torch.int32, device=dev)
    o = torch.empty((s.B, s.Hq, s.dv), dtype=torch.bfloat16, device=dev)
    ws = nsa.workspace(s, nsa.OP_DSA_DECODE, dev)

    def step():
        nsa.dsa_decode(s, hi, di, topk, y["seq_lens"], ix["q_idx"], ix["w_idx"], ix["k_idx"], y["q"], y["k"], y["v"],
                       sel=sel, o=o, ws=ws)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    # the same step with 1 GiB read between steps, so that nothing of the
    # previous step is left in the 256 MB Infinity Cache (median of the steps)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(max(steps, 5))]
    for a, b in ev:
        torch.sum(flush, dim=0, out=acc)
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    cold = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)[len(ev) // 2]
    del flush
    L = s.T
    nbytes = s.B * (L * di * 2 + 2 * L * 4 + min(topk, L) * s.Hkv * (s.dk + s.dv) * 2)
    return {"workload": "DSA-style decode step, bf16 B=32 @65536-token caches, 4 KV x 16 q heads, d_k=192, d_v=128; "
                        "indexer 4 heads x 64, top-2048",
            "us_per_step": round(us, 2), "us_per_step_after_1GiB_read": round(cold, 2),
            "algorithmic_MB": round(nbytes / 1e6, 2),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}


def dsa_prefill(steps, topk=2048, hi=4, di=64):
    """DSA-style attention for every position of T=16384 tokens (its own
    top-2,048), timed apart from the headline step."""
    s = WORKLOADS["bf16_fwdbwd_T16384"].shape
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(1007)
    dt = torch.bfloat16
    qi = (torch.randn((s.B, s.T, hi, di), generator=g, device=dev) / math.sqrt(di)).to(dt)
    wi = (torch.randn((s.B, s.T, hi), generator=g, device=dev) / math.sqrt(hi)).to(dt)
    ki = torch.randn((s.B, s.T, di), generator=g, device=dev).to(dt)
    q = torch.randn((s.B, s.T, s.Hq, s.dk), generator=g, device=dev).to(dt)
    k = torch.randn((s.B, s.Hkv, s.T, s.dk), generator=g, device=dev).to(dt)
    v = torch.randn((s.B, s.Hkv, s.T, s.dv), generator=g, device=dev).to(dt)
    sel = torch.empty((s.B, s.T, topk), dtype=torch.int32, device=dev)
    o = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=dev)
    ws = nsa.workspace(s, nsa.OP_DSA_PREFILL, dev)

    def step():
        nsa.dsa_prefill(s, hi, di, topk, qi, wi, ki, q, k, v, sel=sel, o=o, ws=ws)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = sum(min(t + 1, topk) for t in range(s.T)) * s.B
    flops = s.B * s.T * (s.T + 1) // 2 * hi * di * 2 + pairs * s.Hq * (s.dk + s.dv) * 2
    return {"workload": "DSA-style attention for every position, bf16 T=16384, 4 KV x 16 q heads, d_k=192, d_v=128; "
                        "indexer 4 heads x 64, top-2048 per position",
            "ms": round(ms, 3), "algorithmic_tflop": round(flops / 1e12, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}


def mlp_compress(s, x, steps):
    """The two-layer compression map at the prefill shape (first layer: the
    linear compression kernel with W1; second layer in place), beside the
    linear map, timed apart from the headline step."""
    dev = x["k"].device
    w = make_mlp_weights(s, 1004, dev)
    ck = torch.empty((s.B, s.Hkv, s.n_pad, s.dk), dtype=torch.bfloat16, device=dev)
    cv = torch.empty((s.B, s.Hkv, s.n_pad, s.dv), dtype=torch.bfloat16, device=dev)

    def lin():
        nsa.compress_kv(s, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"], ck, cv)

    def mlp():
        nsa.compress_kv_mlp(s, x["k"], x["v"], x["w_ck"], x["pe_k"], w["w2_k"], x["w_cv"], x["pe_v"], w["w2_v"],
                            ck, cv)

    def timed(f):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    lin_ms, mlp_ms = timed(lin), timed(mlp)
    fl = prefill_flops(s)["compress"]
    fl2 = 2 * s.n_cmp * (s.dk * s.dk + s.dv * s.dv) * s.Hkv * s.B
    return {"workload": "two-layer compression map, bf16 T=65536, 4 KV heads, d_k=192, d_v=128",
            "linear_ms": round(lin_ms, 4), "mlp_ms": round(mlp_ms, 4), "second_layer_ms": round(mlp_ms - lin_ms, 4),
            "mlp_algorithmic_gflop": round((fl + fl2) / 1e9, 3),
            "mlp_tflops": round((fl + fl2) / (mlp_ms * 1e-3) / 1e12, 2)}


def _timed(fn, steps):
    """Mean milliseconds of fn() over `steps` calls, each bracketed by events
    on the current stream (one untimed call first)."""
    fn()
    torch.cuda.synchronize()
    t = []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        fn()
        e[1].record()
        torch.cuda.synchronize()
        t.append(e[0].elapsed_time(e[1]))
    return float(np.mean(t))


def fwd_bwd(steps):
    """Training forward (compression, the three branches, selection, each
    branch's softmax statistics saved) and backward with the forward's
    selection and statistics at T=16384, timed apart from the headline step."""
    w = WORKLOADS["bf16_fwdbwd_T16384"]
    s = w.shape
    dev = torch.device("cuda:0")
    log("setup: fwd+bwd inputs", s)
    x = make_prefill(s, 1005, dev, unit_scaled=w.unit_scaled, with_grad=True)
    ws = nsa.workspace(s, nsa.OP_BACKWARD, dev)
    wsf = nsa.workspace(s, nsa.OP_FORWARD, dev)

    def fwd():
        ck, cv = nsa.compress_kv(s, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"])
        _, saved, idx = nsa.forward_train(s, x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"], want_idx=True,
                                          ws=wsf)
        return ck, cv, idx, saved

    def bwd(ck, cv, idx, saved):
        return nsa.backward(s, x["q"], x["k"], x["v"], ck, cv, x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"],
                            x["w_g"], x["b_g"], idx, x["do"], ws=ws, saved=saved)

    bwd(*fwd())
    torch.cuda.synchronize()
    tf, tb = [], []
    log("timed fwd+bwd", steps)
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        ck, cv, idx, saved = fwd()
        e[1].record()
        bwd(ck, cv, idx, saved)
        e[2].record()
        torch.cuda.synchronize()
        tf.append(e[0].elapsed_time(e[1]))
        tb.append(e[1].elapsed_time(e[2]))
    fms, bms = float(np.mean(tf)), float(np.mean(tb))
    ff, bf = prefill_flops(s)["total"], backward_flops(s)["total"]
    # the backward that recomputes every branch's statistics, and the plain
    # (inference) forward
    rms = _timed(lambda: bwd(ck, cv, idx, None), steps)
    pms = _timed(lambda: nsa.forward(s, x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"], ws=wsf), steps)
    # the same backward with the two-layer compression map (its second layers,
    # the recomputed hidden layers and the ReLU added to the linear map's work)
    wm = make_mlp_weights(s, 1007, dev)
    wsm = nsa.workspace(s, nsa.OP_BACKWARD_MLP, dev)
    ckm, cvm = nsa.compress_kv_mlp(s, x["k"], x["v"], x["w_ck"], x["pe_k"], wm["w2_k"], x["w_cv"], x["pe_v"],
                                   wm["w2_v"])
    _, saved_m = nsa.forward_train(s, x["q"], x["k"], x["v"], ckm, cvm, x["w_g"], x["b_g"], idx_in=idx, ws=wsf)
    mms = _timed(lambda: nsa.backward_mlp(s, x["q"], x["k"], x["v"], ckm, cvm, x["w_ck"], x["pe_k"], wm["w2_k"],
                                          x["w_cv"], x["pe_v"], wm["w2_v"], x["w_g"], x["b_g"], idx, x["do"], ws=wsm,
                                          saved=saved_m), steps)
    return {"workload": "NSA fwd+bwd bf16 T=16384 (B=1, 4 KV x 16 q heads, d_k=192, d_v=128), dO ~ N(0,1)",
            "fwd_ms": round(fms, 3), "bwd_ms": round(bms, 3), "bwd_mlp_map_ms": round(mms, 3),
            "bwd_recompute_ms": round(rms, 3), "fwd_inference_ms": round(pms, 3),
            "bwd_over_fwd": round(bms / fms, 2),
            "fwd_tflops": round(ff / (fms * 1e-3) / 1e12, 2), "bwd_algorithmic_tflop": round(bf / 1e12, 4),
            "bwd_tflops": round(bf / (bms * 1e-3) / 1e12, 2),
            "bwd_mfma_frac": round(bf / (bms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def small_prefill(wname, steps):
    """Throughput of a smaller prefill workload end to end (compression, the
    three branches, selection, gates), timed apart from the headline step."""
    w = WORKLOADS[wname]
    s = w.shape
    dev = torch.device("cuda:0")
    x = make_prefill(s, 1000, dev, unit_scaled=w.unit_scaled)
    ws = nsa.workspace(s, nsa.OP_FORWARD, dev)
    dt = torch.float32 if s.dtype == "fp32" else torch.bfloat16
    ck = torch.empty((s.B, s.Hkv, s.n_pad, s.dk), dtype=dt, device=dev)
    cv = torch.empty((s.B, s.Hkv, s.n_pad, s.dv), dtype=dt, device=dev)
    o = torch.empty((s.B, s.T, s.Hq, s.dv), dtype=dt, device=dev)

    def step():
        nsa.compress_kv(s, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"], ck, cv)
        nsa.forward(s, x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"], o=o, ws=ws)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(steps, 20)
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    fl = prefill_flops(s)["total"]
    return {"workload": w.description, "dtype": s.dtype, "ms": round(ms, 4),
            "tokens_per_s": round(s.B * s.T / (ms * 1e-3), 1), "algorithmic_gflop": round(fl / 1e9, 3),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 3)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(s, x, flops_total, rows_sample=10240, seed=5):
    """The oracle on a bounded sample of the prefill workload: the full
    compression of all tokens plus `rows_sample` query positions drawn
    uniformly (every KV group); extrapolated to the whole workload."""
    from oracle import oracle as orc

    def np64(t):
        return t.detach().to(torch.float64).cpu().numpy()

    k64, v64 = np64(x["k"]), np64(x["v"])
    t0 = time.perf_counter()
    kc = orc.compress(k64, np64(x["w_ck"]), np64(x["pe_k"]), n_out=s.n_pad, round_bf16=True)
    vc = orc.compress(v64, np64(x["w_cv"]), np64(x["pe_v"]), n_out=s.n_pad, round_bf16=True)
    t_cmp = time.perf_counter() - t0
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.integers(0, s.T, rows_sample)).astype(np.int32)
    qr = np64(x["q"][0, torch.from_numpy(rows).long().to(x["q"].device)])
    oc = orc.Cfg(s.B, s.T, s.Hkv, s.G, s.dk, s.dv)
    t0 = time.perf_counter()
    orc.forward_rows(oc, np.zeros_like(rows), rows, qr, kc, vc, k64, v64, np64(x["w_g"]), np64(x["b_g"]))
    t_rows = time.perf_counter() - t0
    est = t_cmp + t_rows * s.T / rows_sample
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": flops_total / est / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "compression of all %d tokens (%.1f s) + %d uniformly drawn query positions x %d KV groups "
                      "(%.1f s), extrapolated to all %d positions: %.0f s for the step"
                      % (s.T, t_cmp, rows_sample, s.Hkv, t_rows, s.T, est),
            "seconds_measured": round(t_cmp + t_rows, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=10240)
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the fwd+bwd T=16384 measurement reported beside the headline line")
    ap.add_argument("--traffic", type=float, default=None,
                    help="HBM bytes per launch of the roofline kernel from FETCH_SIZE/WRITE_SIZE counters")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB once (counter calibration) and exit")
    args = ap.parse_args()
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 4 * n}), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this NSA build has no multi-GPU path (--gpus %d requested)"
              % args.gpus, flush=True)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", flush=True)
        sys.exit(2)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nsa.lib()
    wp = WORKLOADS["bf16_T65536"]
    wd = WORKLOADS["bf16_decode_B32_T65536"]
    sp, sd = wp.shape, wd.shape

    log("setup: prefill inputs", sp)
    x = make_prefill(sp, 1002, dev, unit_scaled=wp.unit_scaled)
    ck = torch.empty((sp.B, sp.Hkv, sp.n_pad, sp.dk), dtype=torch.bfloat16, device=dev)
    cv = torch.empty((sp.B, sp.Hkv, sp.n_pad, sp.dv), dtype=torch.bfloat16, device=dev)
    ocmp = torch.empty((sp.B, sp.T, sp.Hq, sp.dv), dtype=torch.bfloat16, device=dev)
    scores = torch.empty((sp.B, sp.Hkv, sp.T, sp.nb), dtype=torch.float32, device=dev)
    idx = torch.empty((sp.B, sp.Hkv, sp.T, sp.n), dtype=torch.int32, device=dev)
    o = torch.empty((sp.B, sp.T, sp.Hq, sp.dv), dtype=torch.bfloat16, device=dev)
    wss = nsa.workspace(sp, nsa.OP_SPARSE, dev)

    log("setup: decode caches (2 copies)", sd)
    dec = []
    for c in range(2):
        y = make_decode(sd, 1003 + c, dev, unit_scaled=wd.unit_scaled)
        y["ck"], y["cv"] = nsa.compress_kv(sd, y["k"], y["v"], y["w_ck"], y["pe_k"], y["w_cv"], y["pe_v"])
        dec.append(y)
    od = torch.empty((sd.B, sd.Hq, sd.dv), dtype=torch.bfloat16, device=dev)
    idd = torch.empty((sd.B, sd.Hkv, sd.n), dtype=torch.int32, device=dev)
    wsd = nsa.workspace(sd, nsa.OP_DECODE, dev)
    torch.cuda.synchronize()

    # nsa_forward's launches, each on its own: S2 runs with the window half of
    # S4 in one kernel (nsa_compressed_window_attention)
    stages = ["S1_compress", "S2_compressed_attention_and_window", "S3_select", "S4a_pack_kv_blocks",
              "S4c_selected_gate", "decode_step"]
    nst = len(stages)

    def step(i, ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record()
        mark(0)
        nsa.compress_kv(sp, x["k"], x["v"], x["w_ck"], x["pe_k"], x["w_cv"], x["pe_v"], ck, cv)
        mark(1)
        # the launches nsa_forward makes, each timed on its own
        nsa.compressed_window_attention(sp, x["q"], x["k"], x["v"], ck, cv, x["w_g"], x["b_g"], scores, o)
        mark(2)
        nsa.select_topn(sp, scores, idx)
        mark(3)
        nsa.pack_kv_blocks(sp, x["k"], x["v"], wss)
        mark(4)
        nsa.selected_attention(sp, x["q"], x["k"], x["v"], idx, x["w_g"], x["b_g"], o, wss)
        mark(5)
        y = dec[i % 2]
        nsa.decode_step(sd, y["seq_lens"], y["q"], y["k"], y["v"], y["ck"], y["cv"], y["w_g"], y["b_g"], None,
                        od, None, wsd)
        mark(6)

    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(args.steps)]
    log("timed steps", args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(nst)] for e in evs])  # ms
    st_ms = per.mean(axis=0)
    step_ms = float(np.array([e[0].elapsed_time(e[nst]) for e in evs]).mean())

    # decode steps back to back as a serving loop runs them, alternating the
    # two cache copies (2 x 461 MB, more than the 256 MB Infinity Cache, so a
    # step does not find the previous step's bytes cached); median of the steps
    def dec_step(i):
        y = dec[i % 2]
        nsa.decode_step(sd, y["seq_lens"], y["q"], y["k"], y["v"], y["ck"], y["cv"], y["w_g"], y["b_g"], None,
                        od, None, wsd)

    nb2b = max(2 * args.steps, 10)
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nb2b)]
    dec_step(0)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(dev_ev):
        a.record()
        dec_step(i + 1)
        b.record()
    torch.cuda.synchronize()
    dec_b2b_us = sorted(a.elapsed_time(b) * 1e3 for a, b in dev_ev)[nb2b // 2]

    # S2 and the window kernel as the stage-by-stage calls run them on their
    # own (nsa_compressed_attention, then nsa_window_attention on its o_cmp)
    def standalone(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        fn()
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    log("standalone S2 and window kernels", args.steps)
    sa_ms = {"k_cmp_attn_mfma": standalone(lambda: nsa.compressed_attention(sp, x["q"], ck, cv, ocmp, scores)),
             "k_window_mfma": standalone(lambda: nsa.window_attention(sp, x["q"], x["k"], x["v"], ocmp, x["w_g"],
                                                                      x["b_g"], o))}

    fl = prefill_flops(sp)
    prefill_ms = float(st_ms[:nst - 1].sum())
    tflops = fl["total"] / (prefill_ms * 1e-3) / 1e12
    dec_bytes = decode_bytes(sd)
    dec_us = float(st_ms[nst - 1] * 1e3)
    dec_gbps = dec_bytes / (dec_us * 1e-6) / 1e9

    # roofline of the dominant kernel: every stage below is one kernel launch
    # on the stream the events are recorded on (S1 launches its kernel twice,
    # once for K and once for V; the decode step runs two kernels)
    kv_bytes = 2 * sp.B * sp.Hkv * sp.T * (sp.dk + sp.dv)
    win_flop = fl["window"] + fl["gates"] * 2 // 3
    work = {
        "S2_compressed_attention_and_window": ("k_cmp_attn_mfma+window", "mfma", fl["compressed"] + win_flop,
                                               PEAK_BF16_TFLOPS, "TFLOP/s"),
        "S3_select": ("k_select_generic", "hbm", 4 * sp.B * sp.Hkv * sum(t // 64 + 1 for t in range(0, sp.T, 1)) +
                      4 * sp.B * sp.Hkv * sp.T * sp.n, PEAK_HBM_GBPS, "GB/s"),
        "S4a_pack_kv_blocks": ("k_pack_blocks", "hbm", 2 * kv_bytes, PEAK_HBM_GBPS, "GB/s"),
        "S4c_selected_gate": ("k_selected_mfma", "mfma", fl["selected"] + fl["gates"] // 3, PEAK_BF16_TFLOPS,
                              "TFLOP/s"),
    }
    dom = max(work, key=lambda k: st_ms[stages.index(k)])
    kname, bound, units, peak, unit = work[dom]
    dur_s = st_ms[stages.index(dom)] * 1e-3
    achieved = units / dur_s / (1e12 if unit == "TFLOP/s" else 1e9)
    traffic = args.traffic if args.traffic is not None else measured_traffic(kname)
    roof = {"bound": bound, "kernel": kname, "stage": dom, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
            "avg_launch_ms": round(float(dur_s * 1e3), 4), "algorithmic_per_launch": units}
    kernels = {}
    for k, (kn, bd, u, pk, un) in work.items():
        ach = u / (st_ms[stages.index(k)] * 1e-3) / (1e12 if un == "TFLOP/s" else 1e9)
        kernels[kn] = {"ms": round(float(st_ms[stages.index(k)]), 4), "bound": bd, "achieved": round(ach, 2),
                       "unit": un, "frac": round(ach / pk, 4)}
    kernels_standalone = {}
    for kn, flop in (("k_cmp_attn_mfma", fl["compressed"]), ("k_window_mfma", win_flop)):
        ach = flop / (sa_ms[kn] * 1e-3) / 1e12
        kernels_standalone[kn] = {"ms": round(sa_ms[kn], 4), "bound": "mfma", "achieved": round(ach, 2),
                                  "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}

    res = {
        "metric": "NSA fwd TFLOP/s @64k prefill",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "NSA prefill forward bf16 T=65536 (B=1, 4 KV x 16 q heads, d_k=192, d_v=128, "
                               "l=32 d=16 l'=64 n=16 w=512) + NSA decode step bf16 B=32 @65536-token caches",
                   "global_batch": sp.B, "seq_len": sp.T, "parallelism": "single GPU"},
        "prefill_ms": round(prefill_ms, 3),
        "prefill_tokens_per_s": round(sp.T * sp.B / (prefill_ms * 1e-3), 1),
        "prefill_mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "prefill_algorithmic_tflop": round(fl["total"] / 1e12, 4),
        "stage_ms": {k: round(float(v), 4) for k, v in zip(stages, st_ms)},
        "decode_us_per_step": round(dec_us, 2),
        "decode_us_per_step_back_to_back": round(dec_b2b_us, 2),
        "decode_tokens_per_s": round(sd.B / (dec_us * 1e-6), 1),
        "decode_GBps": round(dec_gbps, 1),
        "decode_hbm_frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
        "decode_algorithmic_MB": round(dec_bytes / 1e6, 2),
        "decode_slots_per_group": decode_slots(sd)["total_slots"],
        "decode_gflop": round(decode_flops(sd) / 1e9, 3),
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
        "kernels": kernels,
        "kernels_standalone": kernels_standalone,
    }
    res["prefill_fp32_T1024"] = small_prefill("fp32_T1024", args.steps)
    res["prefill_bf16_T8192"] = small_prefill("bf16_T8192", args.steps)
    res["mlp_compress_T65536"] = mlp_compress(sp, x, args.steps)
    res["dsa_decode_B32_T65536"] = dsa_decode(sd, dec[0], args.steps)
    res["dsa_prefill_T16384"] = None if args.no_backward else dsa_prefill(args.steps)
    res["fwd_bwd_T16384"] = None if args.no_backward else fwd_bwd(args.steps)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(sp, x, fl["total"], rows_sample=args.cpu_rows)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

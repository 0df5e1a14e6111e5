#!/usr/bin/env python3
"""Benchmark of the sparse MoE fine-tuning hot path on one MI355X.

Default workload: one Qwen3-30B-A3B-shaped MoE layer (T=4096 tokens, H=2048,
E=128 experts, top-8, SwiGLU I=768), bf16 activations and expert weights,
fp32 router and Adam state, a fixed seeded 0.5% active mask.  One step =
forward (router, routing, grouping, gate_up + SwiGLU, down + combine), MSE
loss gradient, masked backward (dA, router gradient, dX, masked dW at the
active entries) and SparseAdam (experts) + dense Adam (router).

Also measured (reported beside the step): the RigL scan on 8192 tokens of the
same layer after an int4 -> bf16 resident dequant (forward, dense backward,
global top-0.5%, RigL drop/grow at 30%), and the CPU oracle on a bounded
sample of the step (a baseline, not a target).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse MoE-layer train-step tokens/s (Qwen3-30B-A3B-shaped); RigL scan ms"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_VEC_PEAK_TFLOPS = 157.3   # MI355X fp32 vector, TFLOP/s

# HBM traffic per launch from rocprofv3 counter runs (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch, median over the step's launches) at the
# default workload, with the sources the kernel is built from at that time.
# Counters are scaled by what they read for a plain 1 GiB device copy.  A
# figure whose sources have changed since is reported as null.
FETCH_SCALE = 2.0   # a 1 GiB copy reads 524,300 KiB of FETCH_SIZE
WRITE_SCALE = 1.0   # and 1,048,576 KiB of WRITE_SIZE
# workload -> kernel class -> (fetch KiB, write KiB, sources hash).  masked_dw
# and adam sum the launches of one step (the two SDDMM launches, the plan
# being kept per list; expert + router Adam); dense_dw sums the operand
# staging and the two GEMMs of one scan; topk_fresh sums every launch of the
# scan's first selection (sample, full read, compaction, candidate rounds,
# emit); the grouped GEMMs sum the GEMM and its tail-split reduction.
G = "be7cec260b74c1c3"  # the GEMM sources
COUNTER_TRAFFIC = {
    "qwen3_step": {
        "router_gemm": (8784, 16384, G),
        "gate_up": (470364, 147462, G),
        "down": (221403, 131072, G),
        "da": (317419, 100111, G),
        "dx": (543301, 131072, G),
        "masked_dw": (168794, 12824, "6803601c95aa6e76"),
        "adam": (28622, 123523, "a431573056f07bd3"),
    },
    "qwen3_scan": {
        "dense_dw": (867356, 2883584, G),
        "topk_fresh": (1338699, 102130, "b540280715697c17"),
    },
    "mixtral_step": {
        "router_gemm": (16526, 1024, G),
        "gate_up": (1957473, 749553, G),
        "down": (1176567, 118272, G),
        "da": (2251406, 517255, G),
        "dx": (2479262, 135628, G),
        "masked_dw": (765037, 45343, "6803601c95aa6e76"),
        "adam": (62219, 281414, "a431573056f07bd3"),
    },
    "mixtral_scan": {
        "dense_dw": (4906550, 5636096, G),
        "topk_fresh": (3123063, 220449, "b540280715697c17"),
    },
}
KERNEL_SOURCES = {
    c: ("gemm_mfma.hpp", "gemm_v2.hpp", "lds_dma.hpp", "moe_mfma.hip", "common.hpp", "moe_internal.hpp")
    for c in ("router_gemm", "gate_up", "down", "da", "dx", "dense_dw")
}
KERNEL_SOURCES.update(topk_fresh=("topk.hip", "common.hpp", "moe_internal.hpp"),
                      masked_dw=("masked_dw.hip", "common.hpp", "moe_internal.hpp"),
                      adam=("optim.hip", "common.hpp"))


def sources_sha(kclass):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kclass, ()):
        with open(os.path.join(ROOT, "sparse_fine_tuning_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload, kclass):
    """Scaled HBM bytes per launch of a kernel class in a workload, or None
    when unmeasured or stale."""
    table = COUNTER_TRAFFIC.get(workload, {})
    if kclass not in table or kclass not in KERNEL_SOURCES:
        return None
    fetch_kib, write_kib, sha = table[kclass]
    if sha != sources_sha(kclass):
        return None
    return (fetch_kib * FETCH_SCALE + write_kib * WRITE_SCALE) * 1024.0


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def algorithmic_work(shape, k):
    """Per-launch algorithmic flops and HBM bytes of each kernel class of one
    step: every operand the method must move, counted once."""
    T, H, E, K, I = shape
    S = T * K
    b = 2  # bf16 bytes
    W_gu, W_d = E * 2 * I * H * b, E * H * I * b
    X = T * H * b
    gu, a = S * 2 * I * b, S * I * b
    return {
        "gate_up": (2.0 * S * H * 2 * I, W_gu + X + gu + a),
        "down": (2.0 * S * I * H, W_d + a + X),
        "da": (2.0 * S * H * I, W_d + X + gu + a + gu),
        "dx": (2.0 * S * 2 * I * H, W_gu + gu + X),
        "masked_dw": (2.0 * k * S / E, 2 * X + gu + a + 8 * k),
        "adam": (0.0, 28 * k + 28 * E * H),
        "router_gemm": (2.0 * T * H * E, X + E * H * 4 + T * E * 4),
    }


def roofline_entry(name, flops, nbytes, ms):
    """The binding roofline of a kernel class; for classes with MFMA work also
    its MFMA utilisation next to the ceiling its arithmetic intensity allows
    (min(1, AI / ridge))."""
    ai = flops / nbytes if nbytes else 0.0
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    extra = {}
    if flops:
        extra = dict(mfma_frac=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                     mfma_ceiling=min(1.0, ai / ridge))
    if flops and ai >= ridge:
        ach = flops / (ms * 1e-3) / 1e12
        return dict(kernel=name, bound="mfma", achieved=ach, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=ach / BF16_PEAK_TFLOPS, **extra)
    ach = nbytes / (ms * 1e-3) / 1e9
    return dict(kernel=name, bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=ach / HBM_PEAK_GBS, **extra)


def make_layer(lay_cls, dims, d, idx, act):
    lay = lay_cls(*dims, act=act, device="cuda")
    lay.load(d["X"], d["Wr"], d["W_gu"], d["W_d"], d["tgt"])
    lay.set_active(idx)
    return lay


def time_kernel_classes(capi, lay, classes, lr):
    """Time (ms) of each kernel class in one step (summed over its launches
    in the step), events recorded on the launch stream by the library's
    timing hook."""
    import torch
    out = {}
    for c in classes:
        capi.timer_arm(c, 8)
        lay.train_step(lr=lr, check_skip=False)
        torch.cuda.synchronize()
        ms = capi.timer_read(8)
        out[capi.KERNEL_CLASS_NAMES[c]] = sum(ms)
    capi.timer_arm(-1)
    return out


def practical_hbm_rates(nbytes=2416 * 10 ** 6):
    """What plain device copies reach on this part: a copy (read + write),
    a fill (write) and a sum (read) of an N-byte fp32 buffer (the size of
    the Qwen3-shaped layer's dense gradient), median of 4 after one warm-up.
    Context for the roofline fractions, which stay against the 8 TB/s
    peak."""
    import numpy as np
    import torch
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)

    def timed(fn):
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts[1:]))

    out = dict(bytes=nbytes,
               copy_GBps=2 * nbytes / timed(lambda: b.copy_(a)) / 1e6,
               fill_GBps=nbytes / timed(lambda: b.fill_(1.0)) / 1e6,
               sum_GBps=nbytes / timed(lambda: a.sum()) / 1e6)
    del a, b
    torch.cuda.empty_cache()
    return out


def adam_scatter_ceiling(capi, lay, lr, reps=10):
    """SparseAdam's update of the expert list against a plain scattered write
    of the same list (usaf_scatter of the compact weights back to W at idx,
    which leaves W unchanged), each timed alone in the cache state the step
    leaves it: forward, loss and masked backward, then the timed call; median
    of reps.  The scattered 2-byte writes bound the update, so this is its
    measured ceiling."""
    import numpy as np
    import torch
    k = lay.idx.numel()

    def prelude():
        lay.nonfinite.zero_()
        lay.forward()
        lay.loss_grad()
        lay.backward()

    def adam():
        capi.sparse_adam(lay.act, lay.W, lay.idx, k, lay.dW, lay.m, lay.v, lay.t + 1, lr, 0.9,
                         0.999, 1e-8, lay.nonfinite, None, w_list=lay.w_list)

    def scatter():
        capi.scatter(lay.act, lay.W, lay.idx, k, lay.w_list)

    out = {}
    for name, fn in (("sparse_adam_in_step_ms", adam), ("scatter_in_step_ms", scatter)):
        ts = []
        for _ in range(reps):
            prelude()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        out[name] = float(np.median(ts))
    out["vs_scatter_ceiling"] = out["sparse_adam_in_step_ms"] / out["scatter_in_step_ms"]
    return out


def rigl_scan(capi, synth, layer_mod, d, idx, dims, scan_tokens, repeats=2):
    """int4 resident dequant, then forward + dense backward + RigL on
    `scan_tokens` tokens; returns timings and turnover."""
    import numpy as np
    import torch
    T, H, E, K, I = dims
    log("rigl: quantising expert weights to int4 (input preparation)")
    rows_gu, rows_d = E * 2 * I, E * H
    q_gu, s_gu = [], []
    Wgu2 = d["W_gu"].reshape(rows_gu, H)
    for r0 in range(0, rows_gu, 16384):
        q, s = synth.quantize_int4_g64(Wgu2[r0:r0 + 16384])
        q_gu.append(q); s_gu.append(s)
    Wd2 = d["W_d"].reshape(rows_d, I)
    q_d, s_d = [], []
    for r0 in range(0, rows_d, 65536):
        q, s = synth.quantize_int4_g64(Wd2[r0:r0 + 65536])
        q_d.append(q); s_d.append(s)
    dev = "cuda"
    qg = torch.from_numpy(np.concatenate(q_gu)).to(dev)
    sg = torch.from_numpy(np.concatenate(s_gu).view(np.int16)).to(dev)
    qd = torch.from_numpy(np.concatenate(q_d)).to(dev)
    sd = torch.from_numpy(np.concatenate(s_d).view(np.int16)).to(dev)
    del q_gu, s_gu, q_d, s_d
    Ts = scan_tokens
    X = synth.to_bf16_values(synth.normal((Ts, H), 1.0, 10))
    tgt = synth.to_bf16_values(synth.normal((Ts, H), 1.0, 14))
    lay = layer_mod.SparseMoELayer(Ts, H, E, K, I, act=capi.BF16, device=dev)
    lay.X = torch.from_numpy(X).to(dev).to(torch.bfloat16)
    lay.tgt = torch.from_numpy(tgt).to(dev).to(torch.bfloat16)
    lay.Wr = torch.from_numpy(d["Wr"]).to(dev)
    N = lay.shape.N
    lay.W = torch.empty(N, dtype=torch.bfloat16, device=dev)
    ngu = lay.shape.n_gate_up
    # the pages' own affine group-128 storage of the same weights, timed on
    # random codes (the scan below uses the symmetric g64 copy)
    gen = torch.Generator(device=dev)
    gen.manual_seed(41)
    qa = [torch.randint(0, 256, (r_, c_ // 2), dtype=torch.uint8, device=dev, generator=gen)
          for r_, c_ in ((rows_gu, H), (rows_d, I))]
    sa = [(torch.rand(r_, c_ // 128, device=dev, generator=gen) * 1e-3).to(torch.float16).view(torch.int16)
          for r_, c_ in ((rows_gu, H), (rows_d, I))]
    za = [(torch.rand(r_, c_ // 128, device=dev, generator=gen) * 15).to(torch.float16).view(torch.int16)
          for r_, c_ in ((rows_gu, H), (rows_d, I))]
    for rep in range(2):
        torch.cuda.synchronize()
        capi.timer_arm(capi.K_DEQUANT, 4)
        capi.dequant_affine(qa[0], sa[0], za[0], rows_gu, H, 128, lay.W[:ngu])
        capi.dequant_affine(qa[1], sa[1], za[1], rows_d, I, 128, lay.W[ngu:])
        torch.cuda.synchronize()
        dqa_ms = capi.timer_read(4)
        capi.timer_arm(-1)
    dqa_bytes = sum(x.numel() for x in qa) + 4 * sum(x.numel() for x in sa) + N * 2
    # the forward on the same codes, dequantised as the GEMMs load them,
    # against the forward on their resident copy (just written above)
    w4 = capi.q4_experts(qa[0], sa[0], za[0], qa[1], sa[1], za[1], 128)

    def forwards(ly):
        out = {}
        for name, run in (("resident", lambda: ly.forward()),
                          ("q4_on_load", lambda: capi.moe_forward_q4(ly.shape, ly.X, ly.Wr, w4, ly.Y,
                                                                     ly.state, ly.ws_fwd))):
            ts = []
            for rep in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                run()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            out[name] = float(np.median(ts[1:]))
        return out

    fwd_ms = forwards(lay)
    # the same at the train step's 4096 tokens (the frozen layers of a stack)
    lay_t = layer_mod.SparseMoELayer(T, H, E, K, I, act=capi.BF16, device=dev)
    lay_t.X = lay.X[:T].contiguous()
    lay_t.Wr = lay.Wr
    lay_t.W = lay.W
    fwd_t = forwards(lay_t)
    del lay_t
    log(f"rigl: forward at {Ts} tokens, resident {fwd_ms['resident']:.3f} ms, 4-bit on load "
        f"{fwd_ms['q4_on_load']:.3f} ms; at {T} tokens {fwd_t['resident']:.3f} / "
        f"{fwd_t['q4_on_load']:.3f} ms")
    del qa, sa, za, w4
    # dequant once into the resident bf16 working copy (timed)
    for rep in range(2):
        torch.cuda.synchronize()
        capi.timer_arm(capi.K_DEQUANT, 4)
        capi.dequant_resident(qg, sg, rows_gu, H, 64, lay.W[:ngu])
        capi.dequant_resident(qd, sd, rows_d, I, 64, lay.W[ngu:])
        torch.cuda.synchronize()
        dq_ms = capi.timer_read(4)
        capi.timer_arm(-1)
    dq_bytes = qg.numel() + sg.numel() * 2 + qd.numel() + sd.numel() * 2 + N * 2
    k = idx.size
    r = (3 * k) // 10
    grad = torch.empty(N, dtype=torch.float32, device=dev)
    ws = torch.empty(capi.workspace_size(capi.WS_RIGL, None, N, k), dtype=torch.uint8, device=dev)
    times, stats = [], None
    for rep in range(repeats + 1):
        lay.set_active(idx)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lay.dense_scan(out=grad)
        st = layer_mod.rigl(lay, grad, r, ws=ws)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) * 1e3
        if rep > 0:
            times.append(dt)
        stats = st.cpu().numpy()
        log(f"rigl: scan {rep} {dt:.2f} ms")
    # the counter figures were taken at the default 8192 scan tokens
    parts = scan_parts(capi, layer_mod, lay, idx, grad, r, ws, dims, Ts,
                       "qwen3_scan" if Ts == 8192 else f"qwen3_scan_t{Ts}")
    log(f"rigl: scan parts {json.dumps({c: round(v['ms'], 4) for c, v in parts.items()})}")
    return dict(rigl_scan_ms=float(np.median(times)), scan_tokens=Ts, scan_kernels=parts,
                dequant_ms=float(sum(dq_ms)), dequant_GBps=dq_bytes / (sum(dq_ms) * 1e-3) / 1e9,
                forward_ms_resident=fwd_ms["resident"], forward_ms_q4_on_load=fwd_ms["q4_on_load"],
                forward_ms_at_step_tokens=dict(tokens=T, **fwd_t),
                dequant_affine_g128_ms=float(sum(dqa_ms)),
                dequant_affine_g128_GBps=dqa_bytes / (sum(dqa_ms) * 1e-3) / 1e9,
                turnover_applied=float(stats[1]) / k, turnover_topk_vs_old=float(stats[2]) / k,
                rigl_k=int(k), rigl_r=int(r))


def scan_parts(capi, layer_mod, lay, idx, grad, r, ws, dims, Ts, workload):
    """Time per kernel class inside one RigL scan (HIP events on the launch
    stream, one scan per class): the dense gradient of every expert weight
    (operand staging and the two GEMMs), the fresh top-k of |g| over all N
    (the first selection of the scan), every selection of the reselection,
    and the merges that build the new list.  Each with its roofline: the
    dense dW against max(MFMA time, HBM time) of its algorithmic flops and
    bytes (dW written once, operands read once), the top-k against one read
    of the N fp32 keys."""
    import torch
    T, H, E, K, I = dims
    N = 3 * E * H * I
    S = Ts * K
    out = {}
    for c in (capi.K_DENSE_DW, capi.K_TOPK, capi.K_RIGL_MERGE):
        lay.set_active(idx)
        torch.cuda.synchronize()
        capi.timer_arm(c, 64)
        lay.dense_scan(out=grad)
        layer_mod.rigl(lay, grad, r, ws=ws)
        torch.cuda.synchronize()
        ms = capi.timer_read(64)
        capi.timer_arm(-1)
        name = capi.KERNEL_CLASS_NAMES[c]
        if c == capi.K_TOPK:
            out["topk_fresh"] = dict(ms=ms[0], **roofline_entry("topk_fresh", 0.0, 4.0 * N, ms[0]),
                                     traffic=counter_traffic(workload, "topk_fresh"),
                                     note="one read of the N fp32 keys is the algorithmic bytes")
            out["topk_all"] = dict(ms=sum(ms), launches=len(ms))
        else:
            out[name] = dict(ms=sum(ms), launches=len(ms))
    fl = 2.0 * S * 3 * I * H
    by = 4.0 * N + 2.0 * S * (2 * I + I) + 2.0 * 2 * Ts * H
    ms = out["dense_dw"]["ms"]
    t_roof = max(fl / (BF16_PEAK_TFLOPS * 1e12), by / (HBM_PEAK_GBS * 1e9)) * 1e3
    out["dense_dw"].update(algorithmic_flops=fl, algorithmic_bytes=by, roofline_ms=t_roof,
                           frac=t_roof / ms, mfma_frac=fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                           hbm_frac=by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           traffic=counter_traffic(workload, "dense_dw"))
    return out


def mixtral_layer(capi, synth, layer_mod, steps, lr):
    """The Mixtral-8x7B-shaped layer (T=4096, H=4096, E=8, K=2, I=14336, bf16,
    seeded 0.5% mask): step throughput with per-class rooflines, and one RigL
    scan (dense gradient, global top-0.5%, drop/grow at 30%) on the same
    4096 tokens.  Inputs are drawn on the device with a seeded generator
    (same distributions as the other workloads); the mask is the seeded
    uniform one."""
    import numpy as np
    import torch
    dims = (4096, 4096, 8, 2, 14336)
    T, H, E, K, I = dims
    N = 3 * E * H * I
    k = (N * 5) // 1000
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(20)
    lay = layer_mod.SparseMoELayer(*dims, act=capi.BF16, device=dev)
    lay.X = torch.randn(T, H, generator=gen, device=dev).to(torch.bfloat16)
    lay.tgt = torch.randn(T, H, generator=gen, device=dev).to(torch.bfloat16)
    lay.Wr = torch.randn(E, H, generator=gen, device=dev) * 0.02
    lay.W = (torch.randn(N, generator=gen, device=dev) * 0.02).to(torch.bfloat16)
    lay.mr = torch.zeros_like(lay.Wr)
    lay.vr = torch.zeros_like(lay.Wr)
    idx = synth.random_mask(N, k, 25)
    lay.set_active(idx)
    for _ in range(3):
        lay.train_step(lr=lr, check_skip=False)
    torch.cuda.synchronize()
    classes = [capi.K_ROUTER_GEMM, capi.K_ROUTE, capi.K_GATE_UP, capi.K_DOWN, capi.K_COMBINE_Y,
               capi.K_MSE, capi.K_DA, capi.K_ROUTER_BWD, capi.K_DX, capi.K_COMBINE_DX,
               capi.K_MASKED_DW, capi.K_ADAM]
    per_class = time_kernel_classes(capi, lay, classes, lr)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        lay.train_step(lr=lr, check_skip=False)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    work = algorithmic_work(dims, k)
    kern = {c: dict(ms=per_class[c], traffic=counter_traffic("mixtral_step", c),
                    **roofline_entry(c, *work[c], per_class[c]))
            for c in per_class if c in work and per_class[c] > 0}
    gemm_fl = sum(work[c][0] for c in ("gate_up", "down", "da", "dx"))
    gemm_ms = sum(per_class[c] for c in ("gate_up", "down", "da", "dx"))
    log(f"mixtral: step {ms:.3f} ms -> {T / (ms * 1e-3):.0f} tokens/s; grouped GEMMs "
        f"{gemm_fl / (gemm_ms * 1e-3) / 1e12:.0f} TFLOP/s")
    # one RigL scan on the step batch
    r = (3 * k) // 10
    grad = torch.empty(N, dtype=torch.float32, device=dev)
    ws = torch.empty(capi.workspace_size(capi.WS_RIGL, None, N, k), dtype=torch.uint8, device=dev)
    scans = []
    for rep in range(3):
        lay.set_active(idx)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lay.dense_scan(out=grad)
        st = layer_mod.rigl(lay, grad, r, ws=ws)
        torch.cuda.synchronize()
        if rep:
            scans.append((time.perf_counter() - t0) * 1e3)
    stats = st.cpu().numpy()
    log(f"mixtral: rigl scan {np.median(scans):.2f} ms")
    parts = scan_parts(capi, layer_mod, lay, idx, grad, r, ws, dims, T, "mixtral_scan")
    log(f"mixtral: scan parts {json.dumps({c: round(v['ms'], 4) for c, v in parts.items()})}")
    out = dict(workload="Mixtral-8x7B-shaped single MoE layer sparse train step",
               tokens=T, hidden=H, experts=E, top_k=K, intermediate=I, active_entries=k,
               value=T / (ms * 1e-3), unit="tokens/s", ms_per_step=ms,
               grouped_gemm_tflops=gemm_fl / (gemm_ms * 1e-3) / 1e12,
               grouped_gemm_mfma_frac=gemm_fl / (gemm_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
               step_kernels=kern, rigl_scan_ms=float(np.median(scans)), scan_kernels=parts,
               rigl_k=int(k),
               rigl_r=int(r), turnover_applied=float(stats[1]) / k,
               turnover_topk_vs_old=float(stats[2]) / k)
    del lay, grad, ws
    torch.cuda.empty_cache()
    return out


def stack_run(capi, layers=48, steps=180, reselect_every=50, peak_lr=2e-4):
    """The stacked workload: 48 Qwen3-shaped layers (T=4096 as 8 x 512
    tokens, bf16 experts, fp32 routers and Adam state), a fresh batch every
    step, the importance pass before step 0 and RigL (30%) before steps 50,
    100 and 150, the README's cosine decay from LR_PEAK.  Weights come from
    the workload's per-layer seeds and the batches from its per-step seeds,
    drawn on the device (same distributions as the other workloads); all
    batches are resident before the timed region.  Reports tokens/s over the
    whole run and over the train steps alone, and the reselection costs."""
    import torch
    from sparse_fine_tuning_amd.stack import MoEStack, cosine_lr
    dims = (4096, 2048, 128, 8, 768)
    T, H, E, K, I = dims
    dev = "cuda"
    stk = MoEStack(layers, *dims, act=capi.BF16, device=dev)
    N = stk.shape.N
    k = (N * 5) // 1000
    r = (k * 3) // 10
    ngu = E * 2 * I * H
    g = torch.Generator(device=dev)
    log(f"stack: {layers} layers, drawing weights")
    for l, lay in enumerate(stk.layers):
        g.manual_seed(1000 * (l + 1) + 1)
        lay.W[:ngu].copy_(torch.randn(ngu, generator=g, device=dev) * 0.02)
        g.manual_seed(1000 * (l + 1) + 2)
        lay.W[ngu:].copy_(torch.randn(N - ngu, generator=g, device=dev) * 0.02)
        g.manual_seed(1000 * (l + 1) + 3)
        lay.Wr.copy_(torch.randn(E, H, generator=g, device=dev) * 0.02)
    batches = []
    for t in range(steps):
        g.manual_seed(100 + t)
        X = torch.randn(T, H, generator=g, device=dev).to(torch.bfloat16)
        g.manual_seed(10000 + t)
        batches.append((X, torch.randn(T, H, generator=g, device=dev).to(torch.bfloat16)))
    torch.cuda.synchronize()
    log(f"stack: {steps} steps")
    reselect_ms, turnover, novelty, losses = [], [], [], []
    t0 = time.perf_counter()
    for t in range(steps):
        stk.set_batch(*batches[t])
        if t % reselect_every == 0:
            torch.cuda.synchronize()
            r0 = time.perf_counter()
            if t == 0:
                stk.importance(k)
            else:
                st = stk.rigl(r)
            torch.cuda.synchronize()
            reselect_ms.append((time.perf_counter() - r0) * 1e3)
            if t > 0:
                st = st.cpu().numpy()
                turnover.append(float(st[:, 1].mean()) / k)
                novelty.append(float(st[:, 2].mean()) / k)
        stk.train_step(cosine_lr(t, steps, peak_lr))
        if t % 10 == 0 or t == steps - 1:
            losses.append(float(stk.loss.item()))
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t0
    train_s = total_s - sum(reselect_ms) * 1e-3
    res = dict(
        workload=f"stack of {layers} Qwen3-30B-A3B-shaped MoE layers, {steps} steps",
        layers=layers, steps=steps, tokens_per_step=T,
        tokens_per_s_including_reselection=T * steps / total_s,
        tokens_per_s_train_steps=T * steps / train_s,
        ms_per_step_train=train_s * 1e3 / steps, total_s=total_s,
        reselect_ms=reselect_ms, reselect_ms_per_layer=[m / layers for m in reselect_ms],
        rigl_k=k, rigl_r=r, turnover_applied=turnover, turnover_topk_vs_old=novelty,
        steps_taken=stk.t, skipped_steps=stk.skipped, loss_every_10_steps=losses,
        lr="cosine from 2e-4 to 0 over the run")
    log(f"stack: {res['tokens_per_s_including_reselection']:.0f} tokens/s with reselection, "
        f"{res['tokens_per_s_train_steps']:.0f} without; {res['ms_per_step_train']:.2f} ms per step; "
        f"reselect ms {[round(m, 1) for m in reselect_ms]}")
    del stk, batches
    torch.cuda.empty_cache()
    return res


def host_info():
    """CPU model (lscpu), the threads BLAS uses and NumPy's BLAS build."""
    import subprocess
    import numpy as np
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
    except Exception:  # pragma: no cover
        pass
    cores, blas = len(os.sched_getaffinity(0)), None
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            cores = int(info[0].get("num_threads", cores))
            blas = f"{info[0].get('internal_api')} {info[0].get('version')} " \
                   f"({info[0].get('threading_layer')} threads, {cores})"
    except Exception:  # pragma: no cover
        pass
    if blas is None:
        try:
            cfg = np.show_config(mode="dicts")
            b = cfg.get("Build Dependencies", {}).get("blas", {})
            blas = f"{b.get('name')} {b.get('version')}"
        except Exception:  # pragma: no cover
            blas = "unknown"
    return dict(cpu_model=model, cores=cores, blas=blas, numpy=np.__version__)


def cpu_baseline(d, idx, dims, gpu):
    """The CPU oracle, as it stands, on each workload (a baseline, not a
    target; BLAS threads = the process's CPU affinity).  ``gpu`` holds the
    GPU's figures of the same run for the ratios.  Where the full oracle run
    would take minutes, a stated sample is timed and scaled linearly in what
    its cost is proportional to."""
    import numpy as np
    import usaf_synth as synth
    from oracle import usaf_oracle as O
    T, H, E, K, I = dims
    Rb = O.Rounding(O.BF16, O.CONTRACT)
    tim = lambda f: (lambda t0: (f(), time.perf_counter() - t0))(time.perf_counter())
    out = {}
    z = lambda n: np.zeros(n)

    # tiny fp32 layer: everything (importance pass, then 3 steps)
    tiny = (128, 64, 8, 2, 32)
    td = synth.moe_layer(*tiny, bf16=False)
    R32 = O.Rounding(O.F32, O.CONTRACT)
    tk = O.select_count(3 * 8 * 64 * 32, 5, 100)
    sc, t_imp = tim(lambda: O.importance_topk(
        O.dense_scan(td["X"], td["tgt"], td["Wr"], td["W_gu"], td["W_d"], 2, R32)["g"], tk))
    steps = []
    st = dict(W_gu=td["W_gu"], W_d=td["W_d"], Wr=td["Wr"], m=z(tk), v=z(tk),
              mr=np.zeros_like(td["Wr"]), vr=np.zeros_like(td["Wr"]), t=0)
    for _ in range(3):
        o, dt = tim(lambda: O.train_step(td["X"], td["tgt"], st["Wr"], st["W_gu"], st["W_d"], 2, sc,
                                         st["m"], st["v"], st["mr"], st["vr"], st["t"], 1e-3, 0.9,
                                         0.999, 1e-8, R32))
        gu_, dd_ = O.unflatten(o["W_flat"], O.Shape(*tiny))
        st.update(W_gu=gu_, W_d=dd_, Wr=o["Wr"], m=o["m"], v=o["v"], mr=o["mr"], vr=o["vr"], t=o["t"])
        steps.append(dt)
    out["tiny_fp32"] = dict(importance_pass_s=t_imp, step_s=steps,
                            tokens_per_s=128 / float(np.median(steps)), sample="all of it")
    log(f"cpu baseline: tiny layer importance {t_imp:.2f} s, steps {[round(x, 2) for x in steps]}")

    # Qwen3-shaped layer: 3 full steps on the same batch and mask, median
    steps = []
    for _ in range(3):
        _, dt = tim(lambda: O.train_step(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, idx,
                                         z(idx.size), z(idx.size), np.zeros_like(d["Wr"]),
                                         np.zeros_like(d["Wr"]), 0, 1e-3, 0.9, 0.999, 1e-8, Rb))
        steps.append(dt)
        log(f"cpu baseline: qwen3 step {dt:.1f} s")
    med = float(np.median(steps))
    out["qwen3_step"] = dict(step_s=steps, median_s=med, tokens_per_s=T / med,
                             gpu_ratio=gpu.get("qwen3_tokens_per_s", 0) / (T / med),
                             sample="3 full steps (4096 tokens, 3,019,898 listed entries), median")

    # RigL scan inputs: dequant (1/16 of the rows, scaled), the dense scan on
    # all 8192 tokens, the selection on the first N/8 entries (scaled)
    N = 3 * E * H * I
    rows = E * 2 * I
    q, sc16 = synth.quantize_int4_g64(d["W_gu"].reshape(rows, H)[: rows // 16])
    _, t_dq = tim(lambda: O.dequant_int4(q, sc16))
    t_dq *= 16 * (N / (rows * H))  # the sampled rows hold 1/16 of gate_up, scaled to all N
    Xs = synth.to_bf16_values(synth.normal((8192, H), 1.0, 10))
    tg = synth.to_bf16_values(synth.normal((8192, H), 1.0, 14))
    scan, t_scan = tim(lambda: O.dense_scan(Xs, tg, d["Wr"], d["W_gu"], d["W_d"], K, Rb))
    n8, k8 = N // 8, (N * 5 // 1000) // 8
    g8 = scan["g"][:n8]
    del scan
    _, t_tk = tim(lambda: O.importance_topk(g8, k8))
    old8 = synth.random_mask(n8, k8, 5)
    wsel = d["W_gu"].ravel()[:n8]  # N/8 < the gate_up part
    _, t_rg = tim(lambda: O.rigl_reselect(g8, wsel, old8, z(k8), z(k8), k8, (3 * k8) // 10))
    del g8, wsel
    scan_s = t_scan + 8 * (t_tk + t_rg)
    out["qwen3_dequant_and_scan"] = dict(
        dequant_s=t_dq, scan_s=scan_s, dense_scan_s=t_scan, topk_s=8 * t_tk, rigl_s=8 * t_rg,
        gpu_ratio=scan_s * 1e3 / max(gpu.get("rigl_scan_ms", 0) or 1e-9, 1e-9),
        sample="dequant: 1/16 of the gate_up rows, scaled to all 604M weights; dense scan: all "
               "8192 tokens; top-k and RigL: the first N/8 gradient entries (k/8, r/8), scaled x8")
    log(f"cpu baseline: qwen3 dequant {t_dq:.1f} s (scaled), scan {scan_s:.1f} s")

    # Mixtral-shaped layer: the oracle step at 128 and 256 tokens, each part
    # extrapolated to 4096 tokens along the line through the two (the fixed
    # part, fp64 copies of 0.94e9 expert weights, does not grow with the
    # tokens); the listed gradient on a 40,000-entry sample of the 7,046,430
    # and Adam on the same sample, scaled by entries
    me, mk2, mi, mh = 8, 2, 14336, 4096
    md = synth.moe_layer(256, mh, me, mk2, mi, bf16=True, seeds=(20, 21, 22, 23, 24))
    Nm = 3 * me * mh * mi
    km = Nm * 5 // 1000
    samp = synth.random_mask(Nm, 40000, 25)
    Rm = O.Rounding(O.BF16, O.CONTRACT)
    parts = {}
    for mt in (128, 256):
        Xm, tm = md["X"][:mt], md["tgt"][:mt]
        fw, t_f = tim(lambda: O.moe_forward(Xm, md["Wr"], md["W_gu"], md["W_d"], mk2, Rm))
        (_, dYm), t_l = tim(lambda: O.mse_loss_grad(fw["Y"], tm, Rm))
        bw, t_b = tim(lambda: O.moe_backward(fw, Xm, md["Wr"], md["W_gu"], md["W_d"], dYm, Rm))
        gm, t_g = tim(lambda: O.weight_grads_at(fw, bw, Xm, dYm, samp,
                                                O.Shape(mt, mh, me, mk2, mi), Rm))
        parts[mt] = (t_f + t_l + t_b, t_g)
        del fw, bw
    line = lambda a, b: a + (b - a) * (4096 - 128) / (256 - 128)
    fwbw = line(parts[128][0], parts[256][0])
    grad = line(parts[128][1], parts[256][1]) * (km / samp.size)
    ngu = me * 2 * mi * mh
    f = samp.astype(np.int64)
    w_at = np.where(f < ngu, md["W_gu"].ravel()[np.minimum(f, ngu - 1)],
                    md["W_d"].ravel()[np.maximum(f - ngu, 0)])
    _, t_a = tim(lambda: O.adam_update(w_at, gm, z(samp.size), z(samp.size), 1, 1e-3, 0.9, 0.999,
                                       1e-8, O.BF16, Rm))
    del md
    step_m = fwbw + grad + t_a * (km / samp.size)
    out["mixtral_step"] = dict(
        step_s=step_m, tokens_per_s=4096 / step_m, measured_s={str(t): v for t, v in parts.items()},
        gpu_ratio=(gpu.get("mixtral_tokens_per_s") or 0) / (4096 / step_m),
        sample="forward, loss and backward timed at 128 and 256 tokens and extrapolated along "
               "that line to 4096; the listed gradient likewise on 40,000 of the 7,046,430 "
               "entries, scaled by entries; Adam on the sample, scaled by entries.  The dense RigL "
               "scan over 1.41e9 weights is not timed on the host (its fp64 gradient alone is 11 GB)")
    log(f"cpu baseline: mixtral step {step_m:.1f} s (extrapolated)")

    # the 48-layer stack: extrapolated from the single-layer figures
    per_layer_scan = out["qwen3_dequant_and_scan"]["scan_s"]
    run_s = 180 * 48 * med + 4 * 48 * per_layer_scan
    out["stack48_extrapolated"] = dict(
        extrapolated=True, run_s=run_s, tokens_per_s=180 * 4096 / run_s,
        how="48 layers x 180 steps x the Qwen3 step median, plus 4 reselections x 48 layers x "
            "the Qwen3 scan above (8192 tokens: an upper figure for the stack's 4096, since the "
            "oracle's scan is dominated by its gradient over all N weights); residual adds "
            "neglected")
    info = host_info()
    return dict(value=T / med, unit="tokens/s", cores=info["cores"], kind="oracle",
                sample="Qwen3-shaped layer: median of 3 full oracle train steps (4096 tokens); "
                       "the other workloads under configs", seconds=med, host=info, configs=out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--scan-tokens", type=int, default=8192)
    ap.add_argument("--no-scan", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-mixtral", action="store_true")
    ap.add_argument("--no-stack", action="store_true")
    ap.add_argument("--stack-steps", type=int, default=180,
                    help="steps of the stacked workload (reselection every 50)")
    ap.add_argument("--stack-only", action="store_true",
                    help="only the 48-layer stacked workload (prints its JSON object)")
    ap.add_argument("--mixtral-only", action="store_true",
                    help="only the Mixtral-shaped layer leg (prints its JSON object)")
    ap.add_argument("--scan-only", action="store_true",
                    help="skip the timed train steps; run only the RigL scan (profiling)")
    ap.add_argument("--print-sha", action="store_true",
                    help="print the source hash of each counter-measured kernel class and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is not "
              f"sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    if args.print_sha:
        print(json.dumps({c: sources_sha(c) for c in KERNEL_SOURCES}))
        return

    import numpy as np
    import torch

    if args.calibrate_copy:
        # a plain copy of known size: scales rocprofv3's FETCH_SIZE / WRITE_SIZE
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "copies": 3}), flush=True)
        return

    import usaf_synth as synth
    from sparse_fine_tuning_amd import capi
    from sparse_fine_tuning_amd import layer as layer_mod

    dims = (4096, 2048, 128, 8, 768)
    T, H, E, K, I = dims
    N = 3 * E * H * I
    k = (N * 5) // 1000
    lr = 1e-3
    if args.mixtral_only:
        print(json.dumps({"mixtral": mixtral_layer(capi, synth, layer_mod, 10, lr)}), flush=True)
        return
    if args.stack_only:
        print(json.dumps({"stack": stack_run(capi, steps=args.stack_steps)}), flush=True)
        return
    log("generating the seeded Qwen3-shaped layer")
    d = synth.moe_layer(*dims, bf16=True, seeds=(0, 1, 2, 3, 4))
    idx = synth.random_mask(N, k, 5)
    if args.scan_only:
        log("rigl scan only")
        print(json.dumps({"rigl": rigl_scan(capi, synth, layer_mod, d, idx, dims,
                                            args.scan_tokens)}), flush=True)
        return
    lay = make_layer(layer_mod.SparseMoELayer, dims, d, idx, capi.BF16)
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        lay.train_step(lr=lr, check_skip=False)
    torch.cuda.synchronize()
    classes = [capi.K_ROUTER_GEMM, capi.K_ROUTE, capi.K_GATE_UP, capi.K_DOWN, capi.K_COMBINE_Y,
               capi.K_MSE, capi.K_DA, capi.K_ROUTER_BWD, capi.K_DX, capi.K_COMBINE_DX,
               capi.K_MASKED_DW, capi.K_ADAM]
    per_class = time_kernel_classes(capi, lay, classes, lr)
    work = algorithmic_work(dims, k)
    dominant = max((c for c in per_class if c in work), key=lambda c: per_class[c])
    dom_class = capi.KERNEL_CLASS_NAMES.index(dominant)
    launches_per_step = {"adam": 2, "masked_dw": 1}.get(dominant, 1)
    log(f"per-class ms {json.dumps({c: round(v, 4) for c, v in per_class.items()})}; dominant {dominant}")

    capi.timer_arm(dom_class, args.steps * launches_per_step)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        lay.train_step(lr=lr, check_skip=False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kms = capi.timer_read(args.steps * launches_per_step)
    capi.timer_arm(-1)
    nonfinite = int(lay.nonfinite.item())
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = T / (ms_step * 1e-3)
    kern_ms = sum(kms) / args.steps  # per step: one launch for every GEMM class
    fl, by = work[dominant]
    roof = roofline_entry(dominant, fl, by, kern_ms)
    roof.update(kernel_ms=kern_ms, launches=len(kms), algorithmic_flops=fl,
                algorithmic_bytes=by, traffic=counter_traffic("qwen3_step", dominant),
                traffic_note="rocprofv3 FETCH_SIZE x%.1f + WRITE_SIZE x%.1f per launch"
                             % (FETCH_SCALE, WRITE_SCALE))
    log(f"step {ms_step:.3f} ms -> {value:.0f} tokens/s; {dominant} {kern_ms:.3f} ms")
    step_kernels = {c: dict(ms=per_class[c], traffic=counter_traffic("qwen3_step", c),
                            **roofline_entry(c, *work[c], per_class[c]))
                    for c in per_class if c in work and per_class[c] > 0}
    if "adam" in step_kernels:
        ceil = adam_scatter_ceiling(capi, lay, lr)
        step_kernels["adam"].update(ceil)
        log(f"SparseAdam in-step {ceil['sparse_adam_in_step_ms'] * 1e3:.1f} us against a plain "
            f"scatter of the same list {ceil['scatter_in_step_ms'] * 1e3:.1f} us "
            f"({ceil['vs_scatter_ceiling']:.3f}x)")
    del lay
    torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Qwen3-30B-A3B-shaped single MoE layer sparse train step",
                   "tokens": T, "hidden": H, "experts": E, "top_k": K, "intermediate": I,
                   "active_entries": k, "density": 0.005, "lr": lr},
        "roofline": roof,
        "hbm_practical": practical_hbm_rates(),
        "nonfinite_steps": nonfinite,
        "step_kernels": step_kernels,
    }
    if not args.no_scan:
        log("rigl scan")
        out["rigl"] = rigl_scan(capi, synth, layer_mod, d, idx, dims, args.scan_tokens)
        out["rigl_scan_ms"] = out["rigl"]["rigl_scan_ms"]
        torch.cuda.empty_cache()
    if not args.no_mixtral and not args.scan_only:
        log("mixtral-shaped layer")
        out["mixtral"] = mixtral_layer(capi, synth, layer_mod, 10, lr)
    if not args.no_stack and not args.scan_only:
        log("stacked workload")
        out["stack"] = stack_run(capi, steps=args.stack_steps)
    if not args.no_cpu:
        log("cpu baseline: the oracle on every workload")
        gpu = dict(qwen3_tokens_per_s=value, rigl_scan_ms=out.get("rigl_scan_ms"),
                   mixtral_tokens_per_s=(out.get("mixtral") or {}).get("value"))
        out["cpu_baseline"] = cpu_baseline(d, idx, dims, gpu)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

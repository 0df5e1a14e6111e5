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
# kernel class -> (fetch KiB, write KiB, sources hash); masked_dw and adam sum
# the launches of one step (the two SDDMM launches, the plan being kept per
# list; expert + router Adam)
COUNTER_TRAFFIC = {
    "router_gemm": (8788, 16384, "11dc2d44b399d193"),
    "gate_up": (470321, 147459, "11dc2d44b399d193"),
    "down": (221360, 131072, "11dc2d44b399d193"),
    "da": (338569, 100112, "11dc2d44b399d193"),
    "dx": (632618, 131072, "11dc2d44b399d193"),
    "masked_dw": (169865, 11803, "0dc1c49d496d20e3"),
    "adam": (28636, 124714, "b8332b752cd03a50"),
}
KERNEL_SOURCES = {
    c: ("gemm_mfma.hpp", "gemm_v2.hpp", "lds_dma.hpp", "moe_mfma.hip", "common.hpp", "moe_internal.hpp")
    for c in ("router_gemm", "gate_up", "down", "da", "dx", "dense_dw")
}
KERNEL_SOURCES.update(masked_dw=("masked_dw.hip", "common.hpp", "moe_internal.hpp"),
                      adam=("optim.hip", "common.hpp"))


def sources_sha(kclass):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kclass, ()):
        with open(os.path.join(ROOT, "sparse_fine_tuning_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(kclass):
    """Scaled HBM bytes per launch, or None when unmeasured or stale."""
    if kclass not in COUNTER_TRAFFIC or kclass not in KERNEL_SOURCES:
        return None
    fetch_kib, write_kib, sha = COUNTER_TRAFFIC[kclass]
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
    del qa, sa, za
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
    return dict(rigl_scan_ms=float(np.median(times)), scan_tokens=Ts,
                dequant_ms=float(sum(dq_ms)), dequant_GBps=dq_bytes / (sum(dq_ms) * 1e-3) / 1e9,
                dequant_affine_g128_ms=float(sum(dqa_ms)),
                dequant_affine_g128_GBps=dqa_bytes / (sum(dqa_ms) * 1e-3) / 1e9,
                turnover_applied=float(stats[1]) / k, turnover_topk_vs_old=float(stats[2]) / k,
                rigl_k=int(k), rigl_r=int(r))


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
    kern = {c: dict(ms=per_class[c], **roofline_entry(c, *work[c], per_class[c]))
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
    out = dict(workload="Mixtral-8x7B-shaped single MoE layer sparse train step",
               tokens=T, hidden=H, experts=E, top_k=K, intermediate=I, active_entries=k,
               value=T / (ms * 1e-3), unit="tokens/s", ms_per_step=ms,
               grouped_gemm_tflops=gemm_fl / (gemm_ms * 1e-3) / 1e12,
               grouped_gemm_mfma_frac=gemm_fl / (gemm_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
               step_kernels=kern, rigl_scan_ms=float(np.median(scans)), rigl_k=int(k),
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


def cpu_baseline(d, idx, dims, sample_tokens):
    """The CPU oracle, as it stands, on one train step over a sample of the
    layer's tokens (same weights and mask); tokens/s."""
    import numpy as np
    from oracle import usaf_oracle as O
    T, H, E, K, I = dims
    R = O.Rounding(O.BF16, O.CONTRACT)
    X = d["X"][:sample_tokens]
    tgt = d["tgt"][:sample_tokens]
    z = np.zeros(idx.size)
    t0 = time.perf_counter()
    O.train_step(X, tgt, d["Wr"], d["W_gu"], d["W_d"], K, idx, z, z, np.zeros_like(d["Wr"]),
                 np.zeros_like(d["Wr"]), 0, 1e-3, 0.9, 0.999, 1e-8, R)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max(int(p.get("num_threads", 1)) for p in threadpool_info()) or 1
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    return dict(value=sample_tokens / dt, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"one oracle train step (forward, loss, masked backward, SparseAdam, "
                       f"router Adam) on {sample_tokens} of the {T} tokens of the same layer; "
                       f"{dt:.1f} s", seconds=dt)


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
    ap.add_argument("--cpu-tokens", type=int, default=4096)
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
                algorithmic_bytes=by, traffic=counter_traffic(dominant),
                traffic_note="rocprofv3 FETCH_SIZE x%.1f + WRITE_SIZE x%.1f per launch"
                             % (FETCH_SCALE, WRITE_SCALE))
    log(f"step {ms_step:.3f} ms -> {value:.0f} tokens/s; {dominant} {kern_ms:.3f} ms")
    step_kernels = {c: dict(ms=per_class[c], traffic=counter_traffic(c),
                            **roofline_entry(c, *work[c], per_class[c]))
                    for c in per_class if c in work and per_class[c] > 0}
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
        log(f"cpu baseline: oracle on {args.cpu_tokens} tokens")
        out["cpu_baseline"] = cpu_baseline(d, idx, dims, args.cpu_tokens)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

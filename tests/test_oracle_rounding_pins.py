"""Pins of where the oracle's contract mode rounds.

The oracle's contract mode computes in float64 and rounds at the points where
the GPU stores a narrower type (bf16 or fp32 activations; fp32 logits, routing
weights, weight gradients and moments).  Those points are a reading of the
pages: a bf16 model whose every stored tensor is rounded once.  This file
evaluates one sparse train step a second way, token by token and slot by slot
in torch float64, rounding with torch's own conversions at the points listed
here, and requires the oracle's step to agree bit for bit:

  rounded to the activation dtype: the router weight the forward multiplies
  by (bf16 layers only), g|u, a = silu(g)*u, each slot's expert output y, the
  layer output Y, dY, dGU, each slot's input gradient W_gu^T dGU, dX, and
  the updated expert weights;
  rounded to fp32: logits, routing weights, dw, the router's logit
  gradients, dWr, the listed weight gradients, Adam's m and v, and the
  updated router.

Every other intermediate stays in float64.  The derivative of silu(g)*u is
taken by torch autograd rather than written out.  A second test removes each
rounding call of the oracle's step in turn (one at a time) and requires that
the comparison then fails: no rounding point can move or vanish unnoticed.
"""
import numpy as np
import pytest
import torch

import usaf_synth as synth
from oracle import usaf_oracle as O

LR, B1, B2, EPS = 1e-3, 0.9, 0.999, 1e-8


# --------------------------------------------------------------------------
# roundings by torch's conversions
# --------------------------------------------------------------------------
def r32(x: torch.Tensor) -> torch.Tensor:
    """float64 -> nearest fp32 (torch's conversion rounds to nearest even)."""
    return x.to(torch.float32).to(torch.float64)


def rbf16(x: torch.Tensor) -> torch.Tensor:
    """float64 -> nearest bf16, ties to even.  torch converts float64 to bf16
    through fp32, which can round twice; rounding to fp32 by "round to odd"
    first (truncate, then set the last bit of an inexact result) keeps 16
    more bits than bf16, and a round-to-nearest-even from such a value equals
    the direct rounding (Boldo and Melquiond, "When double rounding is odd")."""
    y = x.to(torch.float32)
    inexact = y.to(torch.float64) != x
    toward_zero = torch.where(y.to(torch.float64).abs() > x.abs(),
                              torch.nextafter(y, torch.zeros_like(y)), y)
    bits = toward_zero.view(torch.int32)
    odd = torch.where(inexact, bits | 1, bits).view(torch.float32)
    return odd.to(torch.bfloat16).to(torch.float64)


def test_rbf16_is_the_nearest_bf16():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000) * 10.0 ** rng.integers(-20, 20, 200000)
    # values just beside bf16 midpoints, where a rounding through fp32 goes wrong
    mids = O.bf16_rne(rng.standard_normal(20000)) * (1 + 2.0 ** -9)
    x = np.concatenate([x, mids, np.nextafter(mids, 0), np.nextafter(mids, 10)])
    got = rbf16(torch.from_numpy(x)).numpy()
    assert np.array_equal(got, O.bf16_rne(x))


# --------------------------------------------------------------------------
# the step, a second way
# --------------------------------------------------------------------------
def entry_of(f, E, H, I):
    """Flat index -> (down?, expert, row, column) by plain division."""
    ngu = E * 2 * I * H
    if f < ngu:
        e, rem = divmod(f, 2 * I * H)
        r, c = divmod(rem, H)
        return False, e, r, c
    e, rem = divmod(f - ngu, H * I)
    r, c = divmod(rem, I)
    return True, e, r, c


def step_by_slots(X, tgt, Wr, W_gu, W_d, K, idx, bf16):
    """One sparse step (forward, MSE, backward, listed gradients, Adam at
    t = 1 from zero moments, dense router Adam), token by token."""
    t64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    X, tgt, Wr, W_gu, W_d = map(t64, (X, tgt, Wr, W_gu, W_d))
    ract = rbf16 if bf16 else r32
    T, H = X.shape
    E, I2, _ = W_gu.shape
    I = I2 // 2
    Wr_used = rbf16(Wr) if bf16 else Wr
    out = {}
    # routing per token
    logits = torch.stack([r32(Wr_used @ X[t]) for t in range(T)])
    ids = torch.zeros(T, K, dtype=torch.int64)
    w = torch.zeros(T, K, dtype=torch.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:K]
        ids[t] = torch.tensor(order)
        sel = logits[t, order]
        z = torch.exp(sel - sel.max())
        w[t] = r32(z / z.sum())
    # experts per slot
    S = T * K
    gu = torch.zeros(S, I2, dtype=torch.float64)
    a = torch.zeros(S, I, dtype=torch.float64)
    Y = torch.zeros(T, H, dtype=torch.float64)
    for t in range(T):
        acc = torch.zeros(H, dtype=torch.float64)
        for j in range(K):
            s, e = t * K + j, int(ids[t, j])
            gu[s] = ract(W_gu[e] @ X[t])
            g, u = gu[s, :I], gu[s, I:]
            a[s] = ract(torch.nn.functional.silu(g) * u)
            y = ract(W_d[e] @ a[s])
            acc = acc + w[t, j] * y
        Y[t] = ract(acc)
    dY = ract(2.0 * (Y - tgt) / Y.numel())
    # backward per slot
    dw = torch.zeros(T, K, dtype=torch.float64)
    dgu = torch.zeros(S, I2, dtype=torch.float64)
    for t in range(T):
        for j in range(K):
            s, e = t * K + j, int(ids[t, j])
            Ud = W_d[e].T @ dY[t]
            dw[t, j] = r32(Ud @ a[s])
            g, u = gu[s, :I], gu[s, I:]
            _, (dg, du) = torch.autograd.functional.vjp(
                lambda gg, uu: torch.nn.functional.silu(gg) * uu, (g, u), w[t, j] * Ud)
            dgu[s] = ract(torch.cat([dg, du]))
    dlogits = torch.zeros(T, E, dtype=torch.float64)
    dWr = torch.zeros(E, H, dtype=torch.float64)
    dX = torch.zeros(T, H, dtype=torch.float64)
    for t in range(T):
        mean_dw = (w[t] * dw[t]).sum()
        xr = torch.zeros(H, dtype=torch.float64)
        for j in range(K):
            e = int(ids[t, j])
            dl = r32(w[t, j] * (dw[t, j] - mean_dw))
            dlogits[t, e] = dl
            xr = xr + dl * Wr_used[e]
        acc = torch.zeros(H, dtype=torch.float64)
        for j in range(K):
            s, e = t * K + j, int(ids[t, j])
            acc = acc + ract(W_gu[e].T @ dgu[s])
        dX[t] = ract(acc + xr)
    for e in range(E):
        dWr[e] = r32(sum(dlogits[t, e] * X[t] for t in range(T)))
    # listed gradients, one entry at a time
    g_list = []
    for f in np.asarray(idx, np.int64):
        down, e, r, c = entry_of(int(f), E, H, I)
        tot = torch.zeros((), dtype=torch.float64)
        for t in range(T):
            for j in range(K):
                if int(ids[t, j]) != e:
                    continue
                s = t * K + j
                tot = tot + (w[t, j] * dY[t, r] * a[s, c] if down else dgu[s, r] * X[t, c])
        g_list.append(r32(tot))
    g = torch.stack(g_list) if g_list else torch.zeros(0, dtype=torch.float64)
    # Adam at t = 1 from zero moments (Kingma and Ba, Algorithm 1)
    def adam(wv, gv, wround):
        m = r32((1 - B1) * gv)
        v = r32((1 - B2) * gv * gv)
        upd = LR * (m / (1 - B1)) / (torch.sqrt(v / (1 - B2)) + EPS)
        return wround(wv - upd), m, v
    flat = torch.cat([W_gu.reshape(-1), W_d.reshape(-1)])
    i64 = torch.from_numpy(np.asarray(idx, np.int64))
    w_sel, m, v = adam(flat[i64], g, ract)
    flat_new = flat.clone()
    flat_new[i64] = w_sel
    Wr_new, mr, vr = adam(Wr, dWr, r32)
    out.update(logits=logits, topk_ids=ids, topk_w=w, gu=gu, a=a, Y=Y, dY=dY, dw=dw, dgu=dgu,
               dlogits=dlogits, dWr=dWr, dX=dX, g=g, m=m, v=v, W_flat=flat_new, Wr=Wr_new,
               mr=mr, vr=vr)
    return {k_: v_.numpy() for k_, v_ in out.items()}


def oracle_step(d, K, idx, bf16):
    R = O.Rounding(O.BF16 if bf16 else O.F32, O.CONTRACT)
    z = np.zeros(len(idx))
    o = O.train_step(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, idx, z, z,
                     np.zeros_like(d["Wr"]), np.zeros_like(d["Wr"]), 0, LR, B1, B2, EPS, R)
    fw, bw = o["fw"], o["bw"]
    return dict(logits=fw["logits"], topk_ids=fw["topk_ids"], topk_w=fw["topk_w"], gu=fw["gu"],
                a=fw["a"], Y=fw["Y"], dY=o["dY"], dw=bw["dw"], dgu=bw["dgu"],
                dlogits=bw["dlogits"], dWr=bw["dWr"], dX=bw["dX"], g=o["g"], m=o["m"], v=o["v"],
                W_flat=o["W_flat"], Wr=o["Wr"], mr=o["mr"], vr=o["vr"])


def mismatches(a, b):
    """Names of the outputs that are not bit-identical."""
    return [k for k in b if not np.array_equal(np.asarray(a[k], np.float64),
                                               np.asarray(b[k], np.float64))]


DIMS = (40, 64, 4, 2, 32)  # T, H, E, K, I


def case(bf16):
    T, H, E, K, I = DIMS
    d = synth.moe_layer(*DIMS, bf16=bf16, seeds=(70, 71, 72, 73, 74))
    # weights large enough that SwiGLU's curvature and the routing weights matter
    for name in ("W_gu", "W_d", "Wr"):
        d[name] = d[name] * 10
        if bf16 and name != "Wr":
            d[name] = synth.to_bf16_values(d[name])
    N = 3 * E * H * I
    idx = synth.random_mask(N, 600, 75)
    return d, K, idx


@pytest.mark.parametrize("bf16", [True, False])
def test_contract_rounding_points_bit_exact(bf16):
    d, K, idx = case(bf16)
    ref = step_by_slots(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, idx, bf16)
    got = oracle_step(d, K, idx, bf16)
    counts = np.bincount(np.asarray(got["topk_ids"]).ravel(), minlength=DIMS[2])
    assert counts.min() > 0, "every expert needs slots for the rounding of its blocks to show"
    assert mismatches(got, ref) == []


@pytest.mark.parametrize("bf16", [True, False])
def test_every_rounding_call_of_the_step_is_pinned(bf16, monkeypatch):
    """Drop one rounding call of the oracle's step at a time (the rounding
    functions are called through the module, so a wrapper sees every call):
    each drop must change an output."""
    d, K, idx = case(bf16)
    ref = step_by_slots(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, idx, bf16)
    real = {"bf16_rne": O.bf16_rne, "f32_rne": O.f32_rne}
    state = {"n": 0, "skip": -1}

    def wrap(name):
        def f(x):
            i = state["n"]
            state["n"] += 1
            if i == state["skip"]:
                return np.asarray(x, dtype=np.float64)
            return real[name](x)
        return f

    for name in real:
        monkeypatch.setattr(O, name, wrap(name))
    oracle_step(d, K, idx, bf16)
    n_calls = state["n"]
    assert n_calls >= 3 * DIMS[2] + 10
    silent = []
    for skip in range(n_calls):
        state.update(n=0, skip=skip)
        if not mismatches(oracle_step(d, K, idx, bf16), ref):
            silent.append(skip)
    assert silent == [], f"rounding calls {silent} of {n_calls} change no output"

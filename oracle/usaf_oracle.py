"""Plain CPU oracle of the USAF sparse MoE fine-tuning step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP path and imports nothing from ``sparse_fine_tuning_amd``; the two
meet only in the seeded input generator ``usaf_synth``.

What is computed, and where the pages say so (usaf README = the method
author's GitHub page "tsuyu122/usaf"):

* sparse native fine-tuning of the real expert weights, about 0.5% of them,
  picked by gradient magnitude (README, intro and "how it works" bullets);
* the router (gating network) trained densely alongside (README, "how it
  works": router bullet; method-comparison table);
* RigL reselection of the active set every 50 steps (README, "how it works":
  sparsity bullet; environment-variable table, RESELECT_EVERY);
* SparseAdam over the selected entries (README, A100 per-operation table);
* 4-bit expert storage dequantised once into resident copies (README, "how it
  works": caching bullet; quantisation recipe);
* NaN steps are skipped (README, RX 6750 XT results table).

The layer's arithmetic (softmax top-k routing renormalised over the k chosen
experts, SwiGLU experts, MSE loss, Adam with the Kingma-Ba bias correction) is
the plain definition of each step, written out in float64.

Modes
-----
``exact``    float64 everywhere, nothing rounded (finite-difference checks).
``contract`` float64 arithmetic, rounded round-to-nearest-even at the points
             where the GPU path stores a narrower type: the activation dtype
             (bf16 or fp32) for g|u, a, Y, dY, dGU, dX and the expert weights;
             fp32 for logits, routing weights, dw, dlogits, router gradients,
             expert-weight gradient values and Adam moments.

Readings where the pages are silent are stated at the function that takes
them.  Every function here is pinned by ``tests/test_oracle_pins.py`` except
the whole-run training outcome, whose published numbers need weights and data
that are not available (parity unpinned for that outcome only).
"""
from __future__ import annotations

import math
from typing import NamedTuple

import numpy as np

F32 = "f32"
BF16 = "bf16"
EXACT = "exact"
CONTRACT = "contract"

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# ----------------------------------------------------------------------------
# Rounding
# ----------------------------------------------------------------------------
def bf16_rne(x) -> np.ndarray:
    """Round to the nearest bf16 value, ties to even; returns float64.

    bf16 keeps 8 significant bits and fp32's exponent range.  For |x| in the
    binade [2^(e-1), 2^e) the spacing of bf16 values is 2^(e-8); below 2^-126
    (subnormals) the spacing stays 2^-133.  ``np.rint`` rounds half to even,
    so rint(x / spacing) * spacing is the correctly rounded result (both
    scalings are exact powers of two).  Results beyond the largest finite bf16
    become +-inf; NaN and +-inf pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x)
    xf = x[fin]
    _, ex = np.frexp(xf)
    ex = np.maximum(ex, -125)
    spacing = np.ldexp(1.0, ex - 8)
    r = np.rint(xf / spacing) * spacing
    over = np.abs(r) > BF16_MAX
    r[over] = np.copysign(np.inf, r[over])
    out[fin] = r
    return out


def f32_rne(x) -> np.ndarray:
    """Round to the nearest fp32 value (numpy's conversion is IEEE RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


class Rounding:
    """Where values are rounded, per mode and activation dtype."""

    def __init__(self, act: str = F32, mode: str = CONTRACT):
        if act not in (F32, BF16) or mode not in (EXACT, CONTRACT):
            raise ValueError((act, mode))
        self.act_dtype = act
        self.mode = mode

    def act(self, x):
        if self.mode == EXACT:
            return np.asarray(x, dtype=np.float64)
        return bf16_rne(x) if self.act_dtype == BF16 else f32_rne(x)

    def f32(self, x):
        if self.mode == EXACT:
            return np.asarray(x, dtype=np.float64)
        return f32_rne(x)


# ----------------------------------------------------------------------------
# Shapes and the flat index space
# ----------------------------------------------------------------------------
class Shape(NamedTuple):
    T: int
    H: int
    E: int
    K: int
    I: int

    @property
    def S(self) -> int:
        return self.T * self.K

    @property
    def n_gate_up(self) -> int:
        return self.E * 2 * self.I * self.H

    @property
    def N(self) -> int:
        return 3 * self.E * self.H * self.I


def n_expert_weights(H: int, E: int, I: int) -> int:
    """Expert weights of one layer: gate_up [E, 2I, H] plus down [E, H, I]
    (usaf README, quantisation recipe: the fused expert tensors)."""
    return 3 * E * H * I


def select_count(N: int, frac_num: int, frac_den: int) -> int:
    """k = floor(frac * N) with frac = frac_num / frac_den, in integers.

    The pages give the fraction (FRAC = 0.005 in the README's env-var table)
    but not how k is rounded; floor is the reading taken here."""
    return (int(N) * int(frac_num)) // int(frac_den)


def split_flat(f, shape: Shape):
    """Flat index -> (tensor, e, r, c).

    Reading: the flat space is [gate_up (E,2I,H) | down (E,H,I)], row-major,
    the storage order of the README's fused expert tensors.  tensor 0 is
    gate_up (rows [0, I) gate, [I, 2I) up); tensor 1 is down."""
    f = np.asarray(f, dtype=np.int64)
    T, H, E, K, I = shape
    ngu = shape.n_gate_up
    is_down = f >= ngu
    g = np.where(is_down, f - ngu, f)
    rows_gu, cols_gu = 2 * I, H
    rows_d, cols_d = H, I
    e = np.where(is_down, g // (rows_d * cols_d), g // (rows_gu * cols_gu))
    r = np.where(is_down, (g // cols_d) % rows_d, (g // cols_gu) % rows_gu)
    c = np.where(is_down, g % cols_d, g % cols_gu)
    return is_down.astype(np.int64), e, r, c


# ----------------------------------------------------------------------------
# a1: int4 -> resident bf16
# ----------------------------------------------------------------------------
def dequant_affine(q_packed: np.ndarray, scale_bits: np.ndarray, zero_bits: np.ndarray,
                   group: int = 128) -> np.ndarray:
    """The pages' own 4-bit storage (usaf README, "how it works": experts read
    in 4-bit HQQ format; its quantisation recipe uses group size 128): an
    affine code per weight, one fp16 scale s and one fp16 zero z per
    ``group`` consecutive input-dim elements, w = (q - z) * s.  The pages give
    no arithmetic precision; the reading taken here: q - z and the product
    are each formed in fp32 (one rounding each), then rounded once to bf16.
    q is an unsigned nibble (0..15), element 2i in the low nibble of byte i.
    Returns float64 values."""
    q_packed = np.asarray(q_packed, dtype=np.uint8)
    rows, half = q_packed.shape
    codes = np.empty((rows, 2 * half), dtype=np.float32)
    codes[:, 0::2] = q_packed & 0x0F
    codes[:, 1::2] = q_packed >> 4
    s = np.repeat(np.asarray(scale_bits, np.uint16).view(np.float16).astype(np.float32), group, axis=1)
    z = np.repeat(np.asarray(zero_bits, np.uint16).view(np.float16).astype(np.float32), group, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (codes - z) * s          # float32 operations, each rounded once
    return bf16_rne(prod.astype(np.float64))


def dequant_int4(q_packed: np.ndarray, scale_bits: np.ndarray, group: int = 64) -> np.ndarray:
    """Resident dequantisation (usaf README, "how it works": caching bullet;
    quantisation recipe), with the storage taken here: symmetric int4 codes,
    two's-complement nibbles, element 2i in the low nibble of byte i, one fp16
    scale per ``group`` consecutive input-dim elements.

    w = bf16(q * s).  q*s is exact in float64 (4-bit by 11-bit significands),
    so the only rounding is the final one to bf16.  Returns float64 values.
    """
    q_packed = np.asarray(q_packed, dtype=np.uint8)
    rows, half = q_packed.shape
    cols = 2 * half
    lo = (q_packed & 0x0F).astype(np.int64)
    hi = (q_packed >> 4).astype(np.int64)
    codes = np.empty((rows, cols), dtype=np.int64)
    codes[:, 0::2] = lo
    codes[:, 1::2] = hi
    codes = np.where(codes >= 8, codes - 16, codes)
    scale = np.asarray(scale_bits, dtype=np.uint16).view(np.float16).astype(np.float64)
    s_full = np.repeat(scale, group, axis=1)
    return bf16_rne(codes.astype(np.float64) * s_full)


# ----------------------------------------------------------------------------
# a2-a4: routing
# ----------------------------------------------------------------------------
def router_weight_used(Wr, R: Rounding) -> np.ndarray:
    """The router weight the forward GEMM multiplies by.  Reading: the fp32
    master copy is rounded to bf16 for bf16 layers (the GEMM runs on bf16
    matrix cores) and used as is for fp32 layers; the backward is
    straight-through (no derivative of the rounding)."""
    Wr = np.asarray(Wr, dtype=np.float64)
    if R.mode == CONTRACT and R.act_dtype == BF16:
        return bf16_rne(Wr)
    return Wr


def router_logits(X, Wr, R: Rounding) -> np.ndarray:
    """logits[t, e] = sum_h X[t, h] * Wr[e, h] (the gating network of the
    README's router bullet), summed in float64, stored fp32."""
    X = np.asarray(X, dtype=np.float64)
    return R.f32(X @ router_weight_used(Wr, R).T)


def route_topk(logits, K: int, R: Rounding):
    """Per token: the K experts with the largest logits, ordered by (logit
    descending, expert id ascending); routing weights = softmax over those K
    logits (a softmax over all experts renormalised over the chosen K gives the
    same numbers).

    Readings: selection on logits rather than probabilities (softmax is
    monotone); ties go to the lowest expert id."""
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    ids = np.empty((T, K), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t]))
        ids[t] = order[:K]
    sel = np.take_along_axis(logits, ids, axis=1)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), R.f32(w)


def group_by_expert(topk_ids, E: int):
    """Token grouping by expert: slot s = t*K + j, stably sorted by expert id
    (so slots of one expert appear in ascending slot order, i.e. ascending
    token order).  Returns counts [E], offsets [E+1], perm [S] (perm[p] = slot
    at expert-major position p)."""
    flat = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    perm = np.argsort(flat, kind="stable")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32)


# ----------------------------------------------------------------------------
# a5-a6: experts and combine
# ----------------------------------------------------------------------------
def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def moe_forward(X, Wr, W_gu, W_d, K: int, R: Rounding) -> dict:
    """One MoE layer forward.

    Each expert is SwiGLU without bias (gate and up projections fused as
    gate_up [2I, H], down [H, I], the README's fused tensors):
    [g | u] = x W_gu^T, a = silu(g) * u, y = a W_d^T.  The layer output is
    Y[t] = sum_j w[t, j] * y[t*K + j], summed in the fixed order j = 0..K-1.
    Routing is dropless (no capacity limit).
    Reading (rounding points): each slot's expert output y is a tensor of the
    activation dtype, as the down projection of a bf16 model outputs bf16;
    the weighted combine over the K slots is summed in higher precision and
    rounded once.

    Arrays indexed by slot id s = t*K + j: gu [S, 2I], a [S, I].
    """
    X = np.asarray(X, dtype=np.float64)
    W_gu = np.asarray(W_gu, dtype=np.float64)
    W_d = np.asarray(W_d, dtype=np.float64)
    T, H = X.shape
    E, I2, _ = W_gu.shape
    I = I2 // 2
    S = T * K
    logits = router_logits(X, Wr, R)
    ids, w = route_topk(logits, K, R)
    counts, offsets, perm = group_by_expert(ids, E)
    gu = np.zeros((S, I2))
    a = np.zeros((S, I))
    y = np.zeros((S, H))
    for e in range(E):
        slots = perm[offsets[e]:offsets[e + 1]].astype(np.int64)
        if slots.size == 0:
            continue
        tok = slots // K
        gu_e = R.act(X[tok] @ W_gu[e].T)
        g, u = gu_e[:, :I], gu_e[:, I:]
        a_e = R.act(g * _sigmoid(g) * u)
        gu[slots] = gu_e
        a[slots] = a_e
        y[slots] = R.act(a_e @ W_d[e].T)
    y3 = y.reshape(T, K, H)
    Yacc = np.zeros((T, H))
    for j in range(K):
        Yacc = Yacc + w[:, j:j + 1] * y3[:, j, :]
    Y = R.act(Yacc)
    return dict(logits=logits, topk_ids=ids, topk_w=w, counts=counts,
                offsets=offsets, perm=perm, gu=gu, a=a, Y=Y, K=K)


# ----------------------------------------------------------------------------
# a7: loss
# ----------------------------------------------------------------------------
def mse_loss_grad(Y, tgt, R: Rounding):
    """loss = mean over all T*H elements of (Y - tgt)^2; dY = 2 (Y - tgt)/(T*H).
    Reading: the regression loss of the tiny workload, used for every layer
    workload (the layer only needs some dY)."""
    Y = np.asarray(Y, dtype=np.float64)
    tgt = np.asarray(tgt, dtype=np.float64)
    diff = Y - tgt
    n = diff.size
    loss = float(np.mean(diff * diff))
    return loss, R.act(2.0 * diff / n)


# ----------------------------------------------------------------------------
# a8-a10: backward through experts, router and input
# ----------------------------------------------------------------------------
def moe_backward(fw: dict, X, Wr, W_gu, W_d, dY, R: Rounding) -> dict:
    """Gradients of the layer (chain rule through moe_forward).

    U_s = W_d[e]^T dY[t(s)];  dw[t, j] = <U_s, a_s>;  da = w U_s;
    with sigma = sigmoid(g): dg = da * u * sigma * (1 + g (1 - sigma)),
    du = da * g * sigma;  dGU = [dg | du].
    Router (softmax over the chosen K, README router bullet): for chosen j,
    dlogits[t, e_j] = w_j (dw_j - sum_m w_m dw_m); zero elsewhere.
    dWr = dlogits^T X (dense, fp32);  dX_r = dlogits Wr_used.
    dX[t] = sum_j W_gu[e_j]^T dGU_{t*K+j} + dX_r[t].
    Reading (rounding points): each slot's input gradient W_gu^T dGU is a
    tensor of the activation dtype (the gate_up projection's input gradient
    in a bf16 model); the sum over the K slots and the router term is taken
    in higher precision and rounded once.
    """
    X = np.asarray(X, dtype=np.float64)
    W_gu = np.asarray(W_gu, dtype=np.float64)
    W_d = np.asarray(W_d, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    T, H = X.shape
    E, I2, _ = W_gu.shape
    I = I2 // 2
    K = fw["K"]
    S = T * K
    perm, offsets = fw["perm"], fw["offsets"]
    w = np.asarray(fw["topk_w"], dtype=np.float64)
    ids = fw["topk_ids"]
    U = np.zeros((S, I))
    for e in range(E):
        slots = perm[offsets[e]:offsets[e + 1]].astype(np.int64)
        if slots.size:
            U[slots] = dY[slots // K] @ W_d[e]
    a, gu = fw["a"], fw["gu"]
    dw = R.f32(np.sum(U * a, axis=1)).reshape(T, K)
    da = w.reshape(S)[:, None] * U
    g, u = gu[:, :I], gu[:, I:]
    sig = _sigmoid(g)
    dg = da * u * sig * (1.0 + g * (1.0 - sig))
    du = da * g * sig
    dgu = R.act(np.concatenate([dg, du], axis=1))
    # router
    swdw = np.sum(w * dw, axis=1, keepdims=True)
    dl_sel = R.f32(w * (dw - swdw))
    dlogits = np.zeros((T, E))
    np.put_along_axis(dlogits, ids.astype(np.int64), dl_sel, axis=1)
    dWr = R.f32(dlogits.T @ X)
    dXr = dlogits @ router_weight_used(Wr, R)
    # input
    V = np.zeros((S, H))
    for e in range(E):
        slots = perm[offsets[e]:offsets[e + 1]].astype(np.int64)
        if slots.size:
            V[slots] = R.act(dgu[slots] @ W_gu[e])
    V3 = V.reshape(T, K, H)
    dXacc = np.zeros((T, H))
    for j in range(K):
        dXacc = dXacc + V3[:, j, :]
    dX = R.act(dXacc + dXr)
    return dict(dw=dw, dgu=dgu, dlogits=dlogits, dWr=dWr, dXr=dXr, dX=dX)


# ----------------------------------------------------------------------------
# a11 / a13: expert-weight gradients, at listed entries or dense
# ----------------------------------------------------------------------------
def _expert_operands(fw, bw, X, dY, e):
    K = fw["K"]
    perm, offsets = fw["perm"], fw["offsets"]
    slots = perm[offsets[e]:offsets[e + 1]].astype(np.int64)
    tok = slots // K
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    ws = np.asarray(fw["topk_w"], dtype=np.float64).reshape(-1)[slots]
    return slots, tok, X[tok], bw["dgu"][slots], ws[:, None] * dY[tok], fw["a"][slots]


def weight_grads_at(fw, bw, X, dY, flat_idx, shape: Shape, R: Rounding) -> np.ndarray:
    """Expert-weight gradient at each listed flat index (the masked backward:
    gradients exist only for the selected subset, README intro and A100
    table).  For gate_up entry (e, r, c): sum over slots s routed to e of
    dGU[s, r] * X[t(s), c].  For down entry (e, r, c): sum over those slots of
    w_s * dY[t(s), r] * a[s, c].  Summed in float64, stored fp32."""
    flat_idx = np.asarray(flat_idx, dtype=np.int64)
    out = np.zeros(flat_idx.size)
    tens, e_of, r_of, c_of = split_flat(flat_idx, shape)
    for e in np.unique(e_of):
        _, _, Xe, dGUe, wdYe, ae = _expert_operands(fw, bw, X, dY, int(e))
        for tsel, left, right in ((0, dGUe, Xe), (1, wdYe, ae)):
            pick = np.nonzero((e_of == e) & (tens == tsel))[0]
            if pick.size == 0 or left.shape[0] == 0:
                continue
            out[pick] = np.einsum("pi,pi->i", left[:, r_of[pick]], right[:, c_of[pick]])
    return R.f32(out)


def weight_grads_dense(fw, bw, X, dY, shape: Shape, R: Rounding) -> np.ndarray:
    """Every expert-weight gradient, flat [N] (the importance / RigL dense
    pass, README "how it works" and A100 table): per expert,
    dW_gu[e] = dGU_e^T X_e and dW_d[e] = (w dY)_e^T a_e, as matrix products."""
    T, H, E, K, I = shape
    dWgu = np.zeros((E, 2 * I, H))
    dWd = np.zeros((E, H, I))
    for e in range(E):
        _, _, Xe, dGUe, wdYe, ae = _expert_operands(fw, bw, X, dY, e)
        dWgu[e] = dGUe.T @ Xe
        dWd[e] = wdYe.T @ ae
    return R.f32(np.concatenate([dWgu.ravel(), dWd.ravel()]))


# ----------------------------------------------------------------------------
# a12: (Sparse)Adam
# ----------------------------------------------------------------------------
def adam_update(w, g, m, v, t: int, lr, beta1, beta2, eps, w_round, R: Rounding):
    """Adam (Kingma & Ba 2015, Algorithm 1) on the listed entries, the
    README's SparseAdam:  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
    mhat = m / (1 - b1^t);  vhat = v / (1 - b2^t);
    w = w - lr * mhat / (sqrt(vhat) + eps).

    Readings: eps is added to sqrt(vhat) (the paper's form); no weight decay
    and no clipping; m and v are stored fp32; the expert weights have no fp32
    master copy, so ``w_round`` (bf16 or fp32) rounds the updated weight.
    ``t`` is the step number after incrementing (>= 1)."""
    if t < 1:
        raise ValueError("t must be >= 1")
    g = np.asarray(g, dtype=np.float64)
    m = R.f32(beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g)
    v = R.f32(beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g)
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    w_new = np.asarray(w, dtype=np.float64) - lr * mhat / (np.sqrt(vhat) + eps)
    if R.mode == CONTRACT:
        w_new = bf16_rne(w_new) if w_round == BF16 else f32_rne(w_new)
    return w_new, m, v


# ----------------------------------------------------------------------------
# a14: global top-k by |grad|
# ----------------------------------------------------------------------------
def topk_order_key(values) -> np.ndarray:
    """uint64 key whose descending order is (|value| descending, index
    ascending).  |value| is taken in fp32; for non-negative IEEE floats the
    bit pattern is monotone in the value, so (bits << 32) | (2^32-1-index)
    orders first by magnitude, then by lowest index."""
    a = np.abs(np.asarray(values, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    idx = np.arange(a.size, dtype=np.uint64)
    return (a << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - idx)


def importance_topk(grad, k: int, exclude=None) -> np.ndarray:
    """The importance phase (README "how it works": the 0.5% with the largest
    gradient magnitude): the k entries ranked first by (|g| descending, flat
    index ascending), returned as ascending uint32 indices.  ``exclude`` (a
    sorted index list) removes entries from consideration (RigL grow)."""
    key = topk_order_key(grad)
    N = key.size
    if exclude is not None and len(exclude):
        cand = np.ones(N, dtype=bool)
        cand[np.asarray(exclude, dtype=np.int64)] = False
        pos = np.nonzero(cand)[0]
        key = key[pos]
    else:
        pos = None
    if k > key.size:
        raise ValueError("k exceeds the number of candidates")
    if k == 0:
        return np.zeros(0, dtype=np.uint32)
    part = np.argpartition(key, key.size - k)[key.size - k:]
    sel = part if pos is None else pos[part]
    return np.sort(sel).astype(np.uint32)


# ----------------------------------------------------------------------------
# a15: RigL drop / grow
# ----------------------------------------------------------------------------
def rigl_reselect(grad, w_flat, S_old, m_old, v_old, k: int, r: int) -> dict:
    """RigL reselection (README "how it works": sparsity bullet; RESELECT_EVERY).

    Drop D: the r active entries with the smallest |w| (ties: lowest index).
    Grow G: the r inactive entries with the largest |g| (ties: lowest index).
    S_new = sort((S_old minus D) union G).  Kept entries carry their Adam
    moments over; grown entries start at zero.  Weights are not changed.

    Readings: "inactive" means outside S_old, so the applied turnover is r/k;
    the README's turnover figure is read as the share of the fresh top-k that
    lies outside S_old, reported as ``topk_new_vs_old``."""
    S_old = np.asarray(S_old, dtype=np.int64)
    if S_old.size != k or r > k:
        raise ValueError("bad k / r")
    w_abs = np.abs(np.asarray(w_flat, dtype=np.float64)[S_old])
    drop_order = np.lexsort((S_old, w_abs))
    D_pos = np.sort(drop_order[:r])
    keep = np.ones(k, dtype=bool)
    keep[D_pos] = False
    kept = S_old[keep]
    G = importance_topk(grad, r, exclude=S_old).astype(np.int64)
    S_new = np.sort(np.concatenate([kept, G]))
    m_old = np.asarray(m_old, dtype=np.float64)
    v_old = np.asarray(v_old, dtype=np.float64)
    m_new = np.zeros(k)
    v_new = np.zeros(k)
    where_kept = np.searchsorted(S_new, kept)
    m_new[where_kept] = m_old[keep]
    v_new[where_kept] = v_old[keep]
    fresh = importance_topk(grad, k).astype(np.int64)
    novelty = int(np.setdiff1d(fresh, S_old, assume_unique=True).size)
    return dict(S_new=S_new.astype(np.uint32), m=m_new, v=v_new,
                dropped=S_old[D_pos].astype(np.uint32), grown=G.astype(np.uint32),
                n_drop=int(r), n_grow=int(G.size), topk_new_vs_old=novelty)


# ----------------------------------------------------------------------------
# One train step, importance pass and RigL scan (sequencing)
# ----------------------------------------------------------------------------
def is_finite_all(*arrays) -> bool:
    return all(np.all(np.isfinite(np.asarray(a, dtype=np.float64))) for a in arrays)


def train_step(X, tgt, Wr, W_gu, W_d, K, idx, m, v, mr, vr, t, lr, beta1, beta2, eps,
               R: Rounding) -> dict:
    """One sparse step: forward, MSE loss, backward, expert-weight gradients at
    the active ``idx`` only, a dense fp32 router gradient, then SparseAdam on the
    experts and dense Adam on the router with the same step count.

    NaN rule (README results table: NaN steps are skipped): if the loss, dY,
    any listed gradient or the router gradient is non-finite, nothing is
    updated and the step count does not advance.
    """
    shape = Shape(X.shape[0], X.shape[1], W_gu.shape[0], K, W_d.shape[2])
    fw = moe_forward(X, Wr, W_gu, W_d, K, R)
    loss, dY = mse_loss_grad(fw["Y"], tgt, R)
    bw = moe_backward(fw, X, Wr, W_gu, W_d, dY, R)
    g = weight_grads_at(fw, bw, X, dY, idx, shape, R)
    out = dict(fw=fw, bw=bw, loss=loss, dY=dY, g=g, skipped=False)
    flat = np.concatenate([np.asarray(W_gu, np.float64).ravel(),
                           np.asarray(W_d, np.float64).ravel()])
    if not is_finite_all([loss], dY, g, bw["dWr"]):
        out.update(skipped=True, W_flat=flat, m=np.asarray(m, np.float64),
                   v=np.asarray(v, np.float64), Wr=np.asarray(Wr, np.float64),
                   mr=np.asarray(mr, np.float64), vr=np.asarray(vr, np.float64), t=t)
        return out
    t_new = t + 1
    w_round = R.act_dtype
    idx64 = np.asarray(idx, dtype=np.int64)
    w_sel, m_new, v_new = adam_update(flat[idx64], g, m, v, t_new, lr, beta1, beta2, eps,
                                      w_round, R)
    flat_new = flat.copy()
    flat_new[idx64] = w_sel
    Wr_new, mr_new, vr_new = adam_update(Wr, bw["dWr"], mr, vr, t_new, lr, beta1, beta2, eps,
                                         F32, R)
    out.update(W_flat=flat_new, m=m_new, v=v_new, Wr=Wr_new, mr=mr_new, vr=vr_new, t=t_new)
    return out


def unflatten(flat, shape: Shape):
    T, H, E, K, I = shape
    ngu = shape.n_gate_up
    return flat[:ngu].reshape(E, 2 * I, H), flat[ngu:].reshape(E, H, I)


def dense_scan(X, tgt, Wr, W_gu, W_d, K, R: Rounding) -> dict:
    """Forward + backward + every expert-weight gradient (importance / RigL
    dense pass)."""
    shape = Shape(X.shape[0], X.shape[1], W_gu.shape[0], K, W_d.shape[2])
    fw = moe_forward(X, Wr, W_gu, W_d, K, R)
    loss, dY = mse_loss_grad(fw["Y"], tgt, R)
    bw = moe_backward(fw, X, Wr, W_gu, W_d, dY, R)
    g = weight_grads_dense(fw, bw, X, dY, shape, R)
    return dict(fw=fw, bw=bw, loss=loss, dY=dY, g=g)


# ----------------------------------------------------------------------------
# The stacked-layer workload: the trainer loop around the step
# ----------------------------------------------------------------------------
# Readings (the pages train a stack of real model layers; the stacked
# workload keeps only the MoE layers):
# * composition: a residual stream with no attention or norm, so layer l+1
#   reads X_{l+1} = round_act(X_l + Y_l); the loss is the MSE of the last
#   output; in the backward the gradient of X_l is round_act(G_{l+1} + dX_l),
#   where dX_l is layer l's own input gradient for output gradient G_{l+1};
# * the learning rate follows the README's cosine decay from LR_PEAK
#   (environment-variable table) over the run's steps, without warm-up, to 0;
# * every layer's active set is chosen from that layer's own gradients, with
#   k = floor(frac * N) per layer (README intro and "how it works": the
#   importance phase; RigL every RESELECT_EVERY steps).


def residual_add(a, b, R: Rounding) -> np.ndarray:
    """The residual stream: round_act(a + b), the sum taken in float64."""
    return R.act(np.asarray(a, dtype=np.float64) + np.asarray(b, dtype=np.float64))


def cosine_lr(step: int, total: int, peak: float) -> float:
    """Cosine decay from ``peak`` at step 0 towards 0 at step ``total`` (README
    environment-variable table: LR_PEAK, cosine decay), no warm-up."""
    return 0.5 * peak * (1.0 + math.cos(math.pi * step / total))


def stack_forward(X0, layers: list, K: int, R: Rounding) -> dict:
    """Forward through the stack.  ``layers[l]`` holds W_gu, W_d and Wr.
    Returns the per-layer forward records and the inputs X_0 .. X_L."""
    Xs = [np.asarray(X0, dtype=np.float64)]
    fws = []
    for lay in layers:
        fw = moe_forward(Xs[-1], lay["Wr"], lay["W_gu"], lay["W_d"], K, R)
        fws.append(fw)
        Xs.append(residual_add(Xs[-1], fw["Y"], R))
    return dict(fws=fws, Xs=Xs)


def stack_backward(fwd: dict, layers: list, GL, R: Rounding) -> dict:
    """Backward from the gradient GL of the last output X_L.  Returns, per
    layer, the backward record and the output gradient dY_l = G_{l+1} that
    layer l's weight gradients are taken against, and the gradient G_0."""
    n = len(layers)
    bws, dYs = [None] * n, [None] * n
    G = np.asarray(GL, dtype=np.float64)
    for l in range(n - 1, -1, -1):
        lay = layers[l]
        bw = moe_backward(fwd["fws"][l], fwd["Xs"][l], lay["Wr"], lay["W_gu"], lay["W_d"], G, R)
        bws[l], dYs[l] = bw, G
        G = residual_add(G, bw["dX"], R)
    return dict(bws=bws, dYs=dYs, G0=G)


def stack_scan_grads(X0, tgt, layers: list, K: int, R: Rounding) -> dict:
    """Dense pass over the stack: every expert-weight gradient of every layer
    (the importance / RigL scan of each layer, taken in one backward)."""
    fwd = stack_forward(X0, layers, K, R)
    loss, GL = mse_loss_grad(fwd["Xs"][-1], tgt, R)
    bwd = stack_backward(fwd, layers, GL, R)
    grads = []
    for l, lay in enumerate(layers):
        shape = Shape(np.shape(X0)[0], np.shape(X0)[1], lay["W_gu"].shape[0], K, lay["W_d"].shape[2])
        grads.append(weight_grads_dense(fwd["fws"][l], bwd["bws"][l], fwd["Xs"][l], bwd["dYs"][l],
                                        shape, R))
    return dict(loss=loss, grads=grads, fwd=fwd, bwd=bwd)


def stack_train_step(X0, tgt, layers: list, K: int, t: int, lr, beta1, beta2, eps,
                     R: Rounding, train_from: int = 0) -> dict:
    """One sparse step of the whole stack.  ``layers[l]`` also holds its active
    list idx and its moments m, v, mr, vr.  Every layer's gradients are taken
    first; if the loss, the last output's gradient, or any layer's listed or
    router gradient is non-finite, no layer is updated and the step count
    stays (README results table: NaN steps are skipped).  Otherwise each
    layer takes SparseAdam on its list and dense Adam on its router with the
    shared step count t + 1.

    ``train_from`` (README environment-variable table: TRAIN_FROM freezes the
    layers below it): the layers below it are frozen -- they need no list or
    moments, their gradients are not taken and they are never updated; only
    the trained layers' gradients enter the NaN rule."""
    fwd = stack_forward(X0, layers, K, R)
    loss, GL = mse_loss_grad(fwd["Xs"][-1], tgt, R)
    bwd = stack_backward(fwd, layers, GL, R)
    gs = [None] * train_from
    finite = is_finite_all([loss], GL)
    for l, lay in enumerate(layers):
        if l < train_from:
            continue
        shape = Shape(np.shape(X0)[0], np.shape(X0)[1], lay["W_gu"].shape[0], K, lay["W_d"].shape[2])
        g = weight_grads_at(fwd["fws"][l], bwd["bws"][l], fwd["Xs"][l], bwd["dYs"][l], lay["idx"],
                            shape, R)
        gs.append(g)
        finite = finite and is_finite_all(g, bwd["bws"][l]["dWr"])
    out = dict(loss=loss, fwd=fwd, bwd=bwd, g=gs, skipped=not finite)
    if not finite:
        out.update(layers=[dict(lay) for lay in layers], t=t)
        return out
    new_layers = [dict(lay) for lay in layers[:train_from]]
    for l, lay in enumerate(layers):
        if l < train_from:
            continue
        shape = Shape(np.shape(X0)[0], np.shape(X0)[1], lay["W_gu"].shape[0], K, lay["W_d"].shape[2])
        flat = np.concatenate([np.asarray(lay["W_gu"], np.float64).ravel(),
                               np.asarray(lay["W_d"], np.float64).ravel()])
        idx64 = np.asarray(lay["idx"], dtype=np.int64)
        w_sel, m_new, v_new = adam_update(flat[idx64], gs[l], lay["m"], lay["v"], t + 1, lr, beta1,
                                          beta2, eps, R.act_dtype, R)
        flat[idx64] = w_sel
        W_gu, W_d = unflatten(flat, shape)
        Wr, mr, vr = adam_update(lay["Wr"], bwd["bws"][l]["dWr"], lay["mr"], lay["vr"], t + 1, lr,
                                 beta1, beta2, eps, F32, R)
        new_layers.append(dict(lay, W_gu=W_gu, W_d=W_d, Wr=Wr, m=m_new, v=v_new, mr=mr, vr=vr))
    out.update(layers=new_layers, t=t + 1)
    return out

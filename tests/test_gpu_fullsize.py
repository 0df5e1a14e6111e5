"""GPU parity at the workloads' full sizes, through the same calls and launch
configuration the benchmark times (SparseMoELayer on one stream).

* Qwen3-30B-A3B-shaped layer step (T=4096, H=2048, E=128, K=8, I=768, bf16,
  seeded 0.5% mask): every output of the step against the full oracle step.
* Mixtral-8x7B-shaped layer step (T=4096, H=4096, E=8, K=2, I=14336, bf16):
  every forward / backward tensor against the oracle, the masked gradient and
  the Adam update on a seeded sample of the active entries.
* RigL scan inputs (int4 g64 -> bf16 dequant, 8192 tokens): the dense
  gradient of every expert weight against the oracle, and the GPU's own
  top-0.5% selection against the oracle's (overlap >= 99.9%).
* Global top-k and RigL at N = 603,979,776 on an identical seeded gradient:
  bit-exact sets and moment remap.

Routing is compared exactly; a token whose routing differs must be a
near-tie in the oracle's logits (K-th vs (K+1)-th gap <= 1e-5 max|logit|),
and such tokens (and the experts they touch) are left out of the float
comparisons that depend on them.
"""
import sys

import numpy as np
import pytest
import torch

import usaf_synth as synth
from oracle import usaf_oracle as O

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL_BF16 = 2e-2
DEV = "cuda"
LR = 1e-3


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def capi():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_fine_tuning_amd import capi as c
    return c


def rel(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    den = np.abs(r).max()
    return float(np.abs(g - r).max() / (den if den > 0 else 1.0))


def npf(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def routing_mismatches(gpu_ids, ref_ids, ref_logits, K):
    """Tokens whose routing differs; each must be a near-tie of the oracle."""
    bad = np.nonzero(np.any(gpu_ids != ref_ids, axis=1))[0]
    scale = np.abs(ref_logits).max()
    for t in bad:
        srt = np.sort(ref_logits[t])[::-1]
        gap = srt[K - 1] - srt[K]
        assert gap <= 1e-5 * scale, f"token {t}: routing differs without a near-tie (gap {gap})"
    return bad


def run_step(capi, d, dims, idx):
    """forward, loss, masked backward (host snapshot), then Adam step 1."""
    from sparse_fine_tuning_amd.layer import SparseMoELayer
    lay = SparseMoELayer(*dims, act=capi.BF16, device=DEV)
    lay.load(d["X"], d["Wr"], d["W_gu"], d["W_d"], d["tgt"])
    lay.set_active(idx)
    W0 = lay.W.clone()
    lay.nonfinite.zero_()
    lay.forward()
    lay.loss_grad()
    lay.backward()
    torch.cuda.synchronize()
    st = lay.st
    out = {k: st[k].cpu().numpy() for k in ("topk_ids", "offsets", "perm", "slot_pos")}
    for k in ("logits", "topk_w", "gu", "a", "dgu", "dw"):
        out[k] = npf(st[k])
    out.update(Y=npf(lay.Y), dY=npf(lay.dY), dX=npf(lay.dX), dWr=npf(lay.dWr), dW=npf(lay.dW),
               loss=float(lay.loss.item()))
    lay.adam(1, LR)
    torch.cuda.synchronize()
    assert int(lay.nonfinite.item()) == 0
    changed = torch.nonzero(lay.W.view(torch.int16) != W0.view(torch.int16)).flatten()
    out["changed"] = changed.cpu().numpy().astype(np.int64)
    del W0
    out.update(m=npf(lay.m), v=npf(lay.v), Wr=npf(lay.Wr), mr=npf(lay.mr), vr=npf(lay.vr))
    out["W_at"] = lambda pos: npf(lay.W[torch.from_numpy(np.asarray(pos, np.int64)).to(DEV)])
    out["layer"] = lay
    return out


def compare_forward_backward(g, fw, bw, ref_loss, ref_dY, dims):
    T, H, E, K, I = dims
    bad = routing_mismatches(g["topk_ids"], fw["topk_ids"], fw["logits"], K)
    say(f"  routing mismatches (near-ties): {bad.size}")
    assert rel(g["logits"], fw["logits"]) <= TOL_BF16
    ok_tok = np.ones(T, dtype=bool)
    ok_tok[bad] = False
    bad_e = np.unique(np.concatenate([g["topk_ids"][bad].ravel(), fw["topk_ids"][bad].ravel()]))
    if bad.size == 0:
        assert np.array_equal(g["offsets"], fw["offsets"])
        assert np.array_equal(g["perm"], fw["perm"])
    assert rel(g["topk_w"][ok_tok], fw["topk_w"][ok_tok]) <= TOL_BF16
    # saved activations are expert-major; compare by slot id
    slots = (np.nonzero(ok_tok)[0][:, None] * K + np.arange(K)).ravel()
    pos = g["slot_pos"][slots]
    for name, ref in (("gu", fw["gu"]), ("a", fw["a"]), ("dgu", bw["dgu"])):
        err = rel(g[name][pos], ref[slots])
        say(f"  {name}: {err:.2e}")
        assert err <= TOL_BF16, name
    for name, gv, rv in (("Y", g["Y"], fw["Y"]), ("dY", g["dY"], ref_dY), ("dX", g["dX"], bw["dX"]),
                         ("dw", g["dw"], bw["dw"])):
        err = rel(gv[ok_tok], rv[ok_tok])
        say(f"  {name}: {err:.2e}")
        assert err <= TOL_BF16, name
    ok_e = np.setdiff1d(np.arange(E), bad_e)
    err = rel(g["dWr"][ok_e], bw["dWr"][ok_e])
    say(f"  dWr: {err:.2e}")
    assert err <= TOL_BF16
    assert abs(g["loss"] - ref_loss) <= TOL_BF16 * abs(ref_loss)
    return bad_e


def check_adam_weights(w_gpu, w_ref, g_ref, w_old):
    """Weights after one Adam step.  At t = 1 the update is lr * g/(|g| + eps),
    about lr * sign(g), so where |g| lies within the gradient tolerance of
    zero the two sides may move the weight in opposite directions: there
    the bound is |dW| <= 2 lr plus one bf16 rounding of each side.  Elsewhere
    the usual relative bound applies."""
    g_ref = np.asarray(g_ref, np.float64)
    sure = np.abs(g_ref) > TOL_BF16 * np.abs(g_ref).max()
    err = rel(w_gpu[sure], w_ref[sure])
    say(f"  W after Adam ({sure.mean():.4f} of entries with a clear gradient sign): {err:.2e}")
    assert err <= TOL_BF16
    ulp = np.abs(np.asarray(w_old, np.float64)) * 2.0 ** -7 + 1e-30
    loose = np.abs(w_gpu[~sure] - w_ref[~sure]) <= 2 * LR * (1 + 1e-3) + 2 * ulp[~sure]
    assert loose.all()


def entries_of_experts(idx, dims, experts):
    """Mask of flat indices that belong to any of ``experts``."""
    T, H, E, K, I = dims
    shape = O.Shape(T, H, E, K, I)
    _, e_of, _, _ = O.split_flat(np.asarray(idx, np.int64), shape)
    return np.isin(e_of, experts)


# --------------------------------------------------------------------------
# Qwen3-shaped layer, full step
# --------------------------------------------------------------------------
def test_qwen3_layer_step_full_size(capi):
    dims = (4096, 2048, 128, 8, 768)
    T, H, E, K, I = dims
    say(f"qwen3 full step dims={dims}")
    d = synth.moe_layer(*dims, bf16=True, seeds=(0, 1, 2, 3, 4))
    N = 3 * E * H * I
    k = O.select_count(N, 5, 1000)
    idx = synth.random_mask(N, k, 5)
    g = run_step(capi, d, dims, idx)
    say("  oracle step")
    R = O.Rounding(O.BF16, O.CONTRACT)
    z = np.zeros(k)
    ref = O.train_step(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, idx, z, z,
                       np.zeros_like(d["Wr"]), np.zeros_like(d["Wr"]), 0, LR, 0.9, 0.999, 1e-8, R)
    bad_e = compare_forward_backward(g, ref["fw"], ref["bw"], ref["loss"], ref["dY"], dims)
    keep = ~entries_of_experts(idx, dims, bad_e)
    for name, gv, rv in (("dW", g["dW"], ref["g"]), ("m", g["m"], ref["m"]), ("v", g["v"], ref["v"])):
        err = rel(gv[keep], rv[keep])
        say(f"  {name}: {err:.2e}")
        assert err <= TOL_BF16, name
    i64 = idx.astype(np.int64)
    w_old = np.concatenate([d["W_gu"].ravel(), d["W_d"].ravel()])[i64]
    check_adam_weights(g["W_at"](idx)[keep], ref["W_flat"][i64][keep], ref["g"][keep], w_old[keep])
    for name in ("Wr", "mr", "vr"):
        assert rel(g[name], ref[name]) <= TOL_BF16, name
    # only listed weights may change
    assert np.isin(g["changed"], idx.astype(np.int64)).all()


# --------------------------------------------------------------------------
# Mixtral-shaped layer: full forward / backward, sampled masked dW and Adam
# --------------------------------------------------------------------------
def test_mixtral_layer_step_full_size(capi):
    dims = (4096, 4096, 8, 2, 14336)
    T, H, E, K, I = dims
    say(f"mixtral full step dims={dims}")
    d = synth.moe_layer(*dims, bf16=True, seeds=(20, 21, 22, 23, 24))
    N = 3 * E * H * I
    k = O.select_count(N, 5, 1000)
    idx = synth.random_mask(N, k, 25)
    g = run_step(capi, d, dims, idx)
    lay = g["layer"]
    # masked gradient equals the dense gradient at the listed entries (any size)
    dense = torch.empty(N, dtype=torch.float32, device=DEV)
    # back to the step's starting weights (Adam has moved W and the router)
    lay.W.copy_(torch.from_numpy(np.concatenate([d["W_gu"].ravel(), d["W_d"].ravel()]))
                .to(DEV).to(torch.bfloat16))
    lay.Wr.copy_(torch.from_numpy(d["Wr"]).to(DEV))
    lay.refresh_list()  # W was written in place
    lay.dense_scan(out=dense)
    torch.cuda.synchronize()
    dense_at = npf(dense[torch.from_numpy(idx.astype(np.int64)).to(DEV)])
    # both paths stage bf16(w * dY); they differ only in fp32 summation order
    assert rel(g["dW"], dense_at) <= 1e-4
    del dense
    torch.cuda.empty_cache()
    say("  oracle forward / backward")
    R = O.Rounding(O.BF16, O.CONTRACT)
    fw = O.moe_forward(d["X"], d["Wr"], d["W_gu"], d["W_d"], K, R)
    loss, dY = O.mse_loss_grad(fw["Y"], d["tgt"], R)
    bw = O.moe_backward(fw, d["X"], d["Wr"], d["W_gu"], d["W_d"], dY, R)
    bad_e = compare_forward_backward(g, fw, bw, loss, dY, dims)
    rng = np.random.default_rng(26)
    pick = np.sort(rng.choice(k, size=40000, replace=False))
    pick = pick[~entries_of_experts(idx[pick], dims, bad_e)]
    sample = idx[pick]
    say(f"  oracle masked dW at {sample.size} sampled entries")
    ref_g = O.weight_grads_at(fw, bw, d["X"], dY, sample, O.Shape(*dims), R)
    err = rel(g["dW"][pick], ref_g)
    say(f"  dW sample: {err:.2e}")
    assert err <= TOL_BF16
    flat_at = np.concatenate([d["W_gu"].ravel(), d["W_d"].ravel()])[sample.astype(np.int64)]
    zs = np.zeros(sample.size)
    w_ref, m_ref, v_ref = O.adam_update(flat_at, ref_g, zs, zs, 1, LR, 0.9, 0.999, 1e-8, O.BF16, R)
    for name, gv, rv in (("m", g["m"][pick], m_ref), ("v", g["v"][pick], v_ref)):
        err = rel(gv, rv)
        say(f"  {name} sample: {err:.2e}")
        assert err <= TOL_BF16, name
    check_adam_weights(g["W_at"](sample), w_ref, ref_g, flat_at)
    assert np.isin(g["changed"], idx.astype(np.int64)).all()


# --------------------------------------------------------------------------
# RigL scan inputs: int4 dequant, dense gradient at 8192 tokens, selection
# --------------------------------------------------------------------------
def quantize_layer(d, dims):
    T, H, E, K, I = dims
    qg, sg = synth.quantize_int4_g64(d["W_gu"].reshape(E * 2 * I, H))
    qd, sd = synth.quantize_int4_g64(d["W_d"].reshape(E * H, I))
    return qg, sg, qd, sd


def test_scan_dense_gradient_and_selection_full_size(capi):
    from sparse_fine_tuning_amd.layer import SparseMoELayer, topk
    dims = (4096, 2048, 128, 8, 768)
    T, H, E, K, I = dims
    Ts = 8192
    say("scan: int4 dequant, dense gradient at 8192 tokens, top-0.5%")
    d = synth.moe_layer(*dims, bf16=True, seeds=(0, 1, 2, 3, 4))
    qg, sg, qd, sd = quantize_layer(d, dims)
    N = 3 * E * H * I
    ngu = E * 2 * I * H
    lay = SparseMoELayer(Ts, H, E, K, I, act=capi.BF16, device=DEV)
    X = synth.to_bf16_values(synth.normal((Ts, H), 1.0, 10))
    tgt = synth.to_bf16_values(synth.normal((Ts, H), 1.0, 14))
    lay.X = torch.from_numpy(X).to(DEV).to(torch.bfloat16)
    lay.tgt = torch.from_numpy(tgt).to(DEV).to(torch.bfloat16)
    lay.Wr = torch.from_numpy(d["Wr"]).to(DEV)
    lay.W = torch.empty(N, dtype=torch.bfloat16, device=DEV)
    to_dev = lambda a, dt=None: torch.from_numpy(a if dt is None else a.view(dt)).to(DEV)
    capi.dequant_resident(to_dev(qg), to_dev(sg, np.int16), E * 2 * I, H, 64, lay.W[:ngu])
    capi.dequant_resident(to_dev(qd), to_dev(sd, np.int16), E * H, I, 64, lay.W[ngu:])
    grad = lay.dense_scan()
    k = O.select_count(N, 5, 1000)
    sel = topk(grad, k)
    torch.cuda.synchronize()
    W_host = lay.W.float().cpu().numpy().astype(np.float64)
    g_host = grad.cpu().numpy().astype(np.float64)
    sel_gpu = sel.cpu().numpy().view(np.uint32)
    ids_gpu = lay.st["topk_ids"].cpu().numpy()
    del lay, grad, sel
    torch.cuda.empty_cache()
    say("  oracle dequant")
    deq = lambda q, s: np.concatenate([O.dequant_int4(q[r:r + 16384], s[r:r + 16384])
                                       for r in range(0, q.shape[0], 16384)])
    W_gu = deq(qg, sg).reshape(E, 2 * I, H)
    W_d = deq(qd, sd).reshape(E, H, I)
    assert np.array_equal(W_host[:ngu], W_gu.ravel()), "dequant differs"
    assert np.array_equal(W_host[ngu:], W_d.ravel()), "dequant differs"
    del W_host
    say("  oracle dense scan")
    R = O.Rounding(O.BF16, O.CONTRACT)
    ref = O.dense_scan(X, tgt, d["Wr"], W_gu, W_d, K, R)
    bad = routing_mismatches(ids_gpu, ref["fw"]["topk_ids"], ref["fw"]["logits"], K)
    say(f"  routing mismatches (near-ties): {bad.size}")
    bad_e = np.unique(np.concatenate([ids_gpu[bad].ravel(), ref["fw"]["topk_ids"][bad].ravel()]))
    shape = O.Shape(Ts, H, E, K, I)
    if bad_e.size:
        _, e_of, _, _ = O.split_flat(np.arange(N, dtype=np.int64), shape)
        keep = ~np.isin(e_of, bad_e)
        err = rel(g_host[keep], ref["g"][keep])
    else:
        err = rel(g_host, ref["g"])
    say(f"  dense gradient: {err:.2e}")
    assert err <= TOL_BF16
    # the oracle's top-k of its own gradient, from its k-th key: entries of
    # larger fp32 |g|, then ties by lowest index
    bits = np.abs(ref["g"].astype(np.float32)).view(np.uint32)
    kth = np.partition(bits, bits.size - k)[bits.size - k]
    n_gt = int(np.count_nonzero(bits > kth))
    tie_idx = np.nonzero(bits == kth)[0][: k - n_gt]
    cut = tie_idx[-1] if tie_idx.size else -1
    sg = sel_gpu.astype(np.int64)
    inside = (bits[sg] > kth) | ((bits[sg] == kth) & (sg <= cut))
    overlap = np.count_nonzero(inside) / k
    say(f"  self-computed selection overlap {overlap:.5f}")
    assert overlap >= 0.999


def topk_set_is_exact(g, sel, k):
    """sel (ascending u32) is the top-k of |g| under (|g| desc, index asc):
    exactly k distinct ascending indices, and every selected entry ranks
    above every unselected one.  Ranking is unique, so this fixes the set."""
    sel = np.asarray(sel, np.int64)
    assert sel.size == k and np.all(np.diff(sel) > 0)
    bits = np.abs(np.asarray(g, np.float32)).view(np.uint32)
    mask = np.zeros(bits.size, dtype=bool)
    mask[sel] = True
    sb = bits[sel]
    lo = sb.min()
    lo_idx = sel[sb == lo].max()            # lowest-ranked selected entry
    ub = bits[~mask]
    if ub.size == 0:
        return
    hi = ub.max()
    hi_idx = np.nonzero(~mask & (bits == hi))[0].min()  # highest-ranked unselected entry
    assert (lo > hi) or (lo == hi and lo_idx < hi_idx), "selection is not the top-k"


def check_rigl(grad, w_flat, S_old, m_old, v_old, S_new, m_new, v_new, stats, sel, k, r):
    """RigL's defining properties on host copies: k ascending entries, r
    dropped and r grown; the dropped are the r active entries of smallest |w|
    and the grown the r best |g| outside S_old (ties: lowest index, both
    compared as fp32 bit patterns); kept moments carried over, grown ones
    zero; the stats count the fresh top-k ``sel`` outside S_old."""
    N = grad.size
    S_old64 = np.asarray(S_old, np.int64)
    assert S_new.size == k and np.all(np.diff(S_new) > 0)
    kept = np.intersect1d(S_new, S_old64, assume_unique=True)
    dropped = np.setdiff1d(S_old64, kept, assume_unique=True)
    grown = np.setdiff1d(S_new, kept, assume_unique=True)
    assert dropped.size == r and grown.size == r
    # drop: the r active entries of smallest |w| (ties: lowest index)
    wb = np.abs(np.asarray(w_flat, np.float32)).view(np.uint32)
    dk = wb[dropped].max()
    dk_idx = dropped[wb[dropped] == dk].max()
    kk = wb[kept].min()
    kk_idx = kept[wb[kept] == kk].min()
    assert dk < kk or (dk == kk and dk_idx < kk_idx), "drop set is not the r smallest |w|"
    del wb
    # grow: the top-r of |g| outside S_old
    gb = np.abs(grad).view(np.uint32)
    outside = np.ones(N, dtype=bool)
    outside[S_old64] = False
    outside[grown] = False
    lo = gb[grown].min()
    lo_idx = grown[gb[grown] == lo].max()
    hi = gb[outside].max()
    hi_idx = np.nonzero(outside & (gb == hi))[0].min()
    assert lo > hi or (lo == hi and lo_idx < hi_idx), "grow set is not the top-r outside S_old"
    del gb, outside
    # moments: kept entries carry theirs, grown entries start at zero
    pos_old = np.searchsorted(S_old64, kept)
    pos_new = np.searchsorted(S_new, kept)
    assert np.array_equal(m_new[pos_new], m_old[pos_old])
    assert np.array_equal(v_new[pos_new], v_old[pos_old])
    pos_g = np.searchsorted(S_new, grown)
    assert not m_new[pos_g].any() and not v_new[pos_g].any()
    assert int(stats[0]) == r and int(stats[1]) == r
    novelty = np.setdiff1d(np.asarray(sel, np.int64), S_old64, assume_unique=True).size
    assert int(stats[2]) == novelty
    return novelty


def run_rigl(capi, dims, w_dev, g_dev, S_old, m_old, v_old, r):
    """usaf_rigl_reselect through the layer (list, moments) on device inputs."""
    from sparse_fine_tuning_amd.layer import SparseMoELayer, rigl
    lay = SparseMoELayer(*dims, act=capi.BF16, device=DEV)
    lay.W = w_dev
    lay.set_active(S_old)
    lay.m.copy_(torch.from_numpy(np.asarray(m_old, np.float32)))
    lay.v.copy_(torch.from_numpy(np.asarray(v_old, np.float32)))
    stats = rigl(lay, g_dev, r).cpu().numpy()
    out = (lay.idx.cpu().numpy().view(np.uint32).astype(np.int64), lay.m.cpu().numpy(),
           lay.v.cpu().numpy(), stats)
    del lay
    return out


def test_topk_and_rigl_full_size(capi):
    """Global top-k and RigL at N = 603,979,776 on a seeded gradient, checked
    by the properties that define them (the oracle's own functions are run
    against the kernels at smaller sizes)."""
    from sparse_fine_tuning_amd.layer import topk
    dims = (4096, 2048, 128, 8, 768)
    T, H, E, K, I = dims
    N = 3 * E * H * I
    k = O.select_count(N, 5, 1000)
    r = (3 * k) // 10
    say(f"top-k and RigL at N={N}, k={k}, r={r}")
    w_flat = synth.to_bf16_values(synth.normal((N,), 0.02, 33))
    grad = synth.normal((N,), 1e-6, 30)
    S_old = synth.random_mask(N, k, 5)
    m_old = synth.normal((k,), 1e-7, 31)
    v_old = np.abs(synth.normal((k,), 1e-13, 32))
    g_dev = torch.from_numpy(grad).to(DEV)
    sel = topk(g_dev, k).cpu().numpy().view(np.uint32)
    say("  top-k properties")
    topk_set_is_exact(grad, sel, k)
    w_dev = torch.from_numpy(w_flat).to(DEV).to(torch.bfloat16)
    S_new, m_new, v_new, stats = run_rigl(capi, (8, H, E, K, I), w_dev, g_dev, S_old, m_old,
                                          v_old, r)
    del g_dev, w_dev
    torch.cuda.empty_cache()
    say("  RigL properties")
    check_rigl(grad, w_flat, S_old, m_old, v_old, S_new, m_new, v_new, stats, sel, k, r)


@pytest.mark.parametrize("grow_from", ["fresh_topk", "exclusion_select"])
def test_topk_and_rigl_mixtral_size(capi, grow_from):
    """Top-k and RigL over every expert weight of the Mixtral-shaped layer,
    N = 1,409,286,144 > 2^30 (k = 7,046,430, r = 2,113,929), by the
    defining properties.  Two gradients force the two ways RigL finds its
    grow set: a plain seeded gradient with a random old list (at least r of
    the fresh top-k lie outside the old list: the grow set comes from the
    fresh top-k), and one whose top-k is a known seeded set P with the old
    list holding all of P but r/2 (fewer than r outside: the grow set needs
    a full selection that excludes the old list)."""
    from sparse_fine_tuning_amd.layer import topk
    dims = (8, 4096, 8, 2, 14336)
    _, H, E, K, I = dims
    N = 3 * E * H * I
    k = O.select_count(N, 5, 1000)
    r = (3 * k) // 10
    assert (N, k, r) == (1409286144, 7046430, 2113929)
    say(f"top-k and RigL at N={N}, k={k}, r={r}, grow from {grow_from}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(80)
    g_dev = torch.randn(N, generator=gen, device=DEV) * 1e-6
    if grow_from == "fresh_topk":
        S_old = synth.random_mask(N, k, 81)
    else:
        P = synth.random_mask(N, k, 82)
        P_dev = torch.from_numpy(P.astype(np.int64)).to(DEV)
        big = (1.0 + torch.rand(k, generator=gen, device=DEV)) * 1e-3
        sign = torch.where(torch.rand(k, generator=gen, device=DEV) < 0.5, -1.0, 1.0)
        g_dev[P_dev] = big * sign
        del P_dev, big, sign
        rng = np.random.default_rng(83)
        out_of_P = np.sort(rng.choice(k, size=r // 2, replace=False))
        kept_P = np.delete(P, out_of_P)
        extra = np.setdiff1d(synth.random_mask(N, r, 84), P, assume_unique=True)[: r // 2]
        S_old = np.sort(np.concatenate([kept_P, extra])).astype(np.uint32)
        assert S_old.size == k and np.unique(S_old).size == k
    m_old = synth.normal((k,), 1e-7, 85)
    v_old = np.abs(synth.normal((k,), 1e-13, 86))
    w_dev = (torch.randn(N, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    sel = topk(g_dev, k).cpu().numpy().view(np.uint32)
    grad = g_dev.cpu().numpy()
    say("  top-k properties")
    topk_set_is_exact(grad, sel, k)
    if grow_from == "exclusion_select":
        assert np.array_equal(sel, P), "the top-k of the planted gradient is P"
    S_new, m_new, v_new, stats = run_rigl(capi, dims, w_dev, g_dev, S_old, m_old, v_old, r)
    w_flat = w_dev.float().cpu().numpy()
    del g_dev, w_dev
    torch.cuda.empty_cache()
    say("  RigL properties")
    novelty = check_rigl(grad, w_flat, S_old, m_old, v_old, S_new, m_new, v_new, stats, sel, k, r)
    say(f"  fresh top-k outside the old list: {novelty} (r = {r})")
    assert (novelty >= r) == (grow_from == "fresh_topk")

"""GPU parity of the stacked-layer workload (a residual stack of MoE layers
trained sparsely, importance pass and RigL per layer) against the oracle's
stack functions, and the 48-layer Qwen3-shaped stack at its full size checked
through properties that hold at any size."""
import sys

import numpy as np
import pytest
import torch

import usaf_synth as synth
from oracle import usaf_oracle as O

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2
DEV = "cuda"


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


def npu32(t):
    return t.detach().cpu().numpy().view(np.uint32)


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


# --------------------------------------------------------------------------
# the loss gradient: 16-byte path and element path
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,H", [(64, 192), (33, 64)])
def test_mse_grad_vector_and_element_paths(capi, T, H):
    """Aligned bf16 operands take the 16-byte path, operands one element off
    alignment the element path; dY is the same element-wise arithmetic on
    both (bit-identical), the loss differs only in summation order.  Both
    against the oracle's loss and gradient."""
    say(f"mse_grad T={T} H={H}")
    n = T * H
    Y = synth.to_bf16_values(synth.normal((T, H), 1.0, 900 + T))
    tgt = synth.to_bf16_values(synth.normal((T, H), 1.0, 901 + T))
    shape = capi.Shape(T, H, 4, 2, 32, capi.BF16)
    ws = torch.empty(capi.workspace_size(capi.WS_FORWARD, shape), dtype=torch.uint8, device=DEV)
    out = {}
    for shift in (0, 1):
        yb = torch.zeros(n + 8, dtype=torch.bfloat16, device=DEV)
        tb = torch.zeros(n + 8, dtype=torch.bfloat16, device=DEV)
        db = torch.zeros(n + 8, dtype=torch.bfloat16, device=DEV)
        yb[shift:shift + n] = to_dev(Y, torch.bfloat16).reshape(-1)
        tb[shift:shift + n] = to_dev(tgt, torch.bfloat16).reshape(-1)
        loss = torch.zeros(1, dtype=torch.float32, device=DEV)
        nf = torch.zeros(1, dtype=torch.int32, device=DEV)
        capi.mse_grad(shape, yb[shift:], tb[shift:], db[shift:], loss, nf, ws)
        torch.cuda.synchronize()
        out[shift] = (float(loss.item()), db[shift:shift + n].clone(), int(nf.item()))
    ref_loss, ref_dY = O.mse_loss_grad(Y, tgt, O.Rounding(O.BF16, O.CONTRACT))
    assert np.array_equal(out[0][1].view(torch.int16).cpu().numpy(),
                          out[1][1].view(torch.int16).cpu().numpy())
    for shift in (0, 1):
        lo, dY, nf = out[shift]
        assert nf == 0
        assert abs(lo - ref_loss) <= 1e-5 * ref_loss
        assert rel(npf(dY).reshape(T, H), ref_dY) <= TOL_BF16


# --------------------------------------------------------------------------
# the residual stream
# --------------------------------------------------------------------------
@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("n,shift", [(0, 0), (5, 0), (1000003, 0), (1 << 20, 0), (1 << 20, 1)])
def test_residual_add_bit_exact(capi, act, n, shift):
    """Vector path (n a multiple of 8, 16-byte aligned) and element path
    (ragged n, or operands one element off alignment)."""
    say(f"residual_add act={act} n={n} shift={shift}")
    dt = torch.bfloat16 if act == capi.BF16 else torch.float32
    R = O.Rounding(O.BF16 if act == capi.BF16 else O.F32, O.CONTRACT)
    rng = np.random.default_rng(n + 3)
    # magnitudes spread over 2^-30 .. 2^10 so that some sums are exact, some
    # round, and some are dominated entirely by one side
    a = R.act(rng.standard_normal(n) * 2.0 ** rng.integers(-30, 10, n))
    b = R.act(rng.standard_normal(n) * 2.0 ** rng.integers(-30, 10, n))
    ta = to_dev(np.concatenate([np.zeros(shift), a]), dt)[shift:]
    tb = to_dev(np.concatenate([np.zeros(shift), b]), dt)[shift:]
    out = torch.empty(n + shift, dtype=dt, device=DEV)[shift:]
    capi.residual_add(act, ta, tb, out, n)
    want = O.residual_add(a, b, R)
    assert np.array_equal(npf(out), want)
    capi.residual_add(act, ta, tb, ta, n)  # in place
    assert np.array_equal(npf(ta), want)


def test_residual_add_refusals(capi):
    t = torch.zeros(8, device=DEV)
    with pytest.raises(capi.UsafError):
        capi.residual_add(7, t, t, t, 8)
    with pytest.raises(capi.UsafError):
        capi.residual_add(capi.F32, t, t, t, -1)
    capi.residual_add(capi.F32, None, None, None, 0)


# --------------------------------------------------------------------------
# the stacked train step
# --------------------------------------------------------------------------
def make_layers(L, dims, seed0, bf16):
    T, H, E, K, I = dims
    layers = []
    for l in range(L):
        d = synth.moe_layer(*dims, bf16=bf16, seeds=tuple(seed0 + 1000 * (l + 1) + i for i in range(5)))
        layers.append(dict(W_gu=d["W_gu"], W_d=d["W_d"], Wr=d["Wr"]))
    return layers


def test_stack_checkpoint_resume_bit_exact(capi, tmp_path):
    """A stack saved after the importance pass, two steps, a RigL pass and one
    more step, then resumed from the file onto a fresh stack holding only the
    base weights, repeats the next two steps bit for bit (losses, touched
    weights, lists, moments, router); the expert load of a forward sums to
    T*K per layer."""
    from sparse_fine_tuning_amd.stack import MoEStack, cosine_lr
    dims = (200, 256, 8, 2, 96)
    T, H, E, K, I = dims
    L = 3
    say(f"stack checkpoint L={L} dims={dims}")
    layers = make_layers(L, dims, 7, bf16=True)
    N = 3 * E * H * I
    k = O.select_count(N, 5, 1000)
    r = (3 * k) // 10

    def fresh():
        stk = MoEStack(L, *dims, act=capi.BF16, device=DEV)
        for l, lay in enumerate(layers):
            stk.load_layer(l, lay["W_gu"], lay["W_d"], lay["Wr"])
        return stk

    def batch(t):
        return (synth.to_bf16_values(synth.normal((T, H), 1.0, 300 + t)),
                synth.to_bf16_values(synth.normal((T, H), 1.0, 30000 + t)))

    total = 6
    a = fresh()
    a.set_batch(*batch(0))
    a.importance(k)
    for t in range(4):
        a.set_batch(*batch(t))
        if t == 2:
            a.rigl(r)
        a.train_step(cosine_lr(t, total, 2e-4))
    load = a.expert_load()
    assert load.shape == (L, E) and bool((load.sum(dim=1) == T * K).all())
    ck = str(tmp_path / "stack.safetensors")
    a.save(ck)
    assert all(lay.touched.numel() > k for lay in a.layers)  # RigL grew new entries
    b = fresh()
    b.load(ck)
    assert b.t == a.t == 4
    for t in range(4, total):
        for stk in (a, b):
            stk.set_batch(*batch(t))
            stk.train_step(cosine_lr(t, total, 2e-4))
        torch.cuda.synchronize()
        assert float(a.loss.item()) == float(b.loss.item()), t
    assert a.t == b.t == total
    for la, lb in zip(a.layers, b.layers):
        assert torch.equal(la.W.view(torch.int16), lb.W.view(torch.int16))
        for x, y in ((la.idx, lb.idx), (la.m, lb.m), (la.v, lb.v), (la.Wr, lb.Wr), (la.mr, lb.mr),
                     (la.vr, lb.vr), (la.touched, lb.touched)):
            assert torch.equal(x, y)


def test_bf16_stack_steps_vs_oracle(capi):
    """Three layers, fixed 0.5% masks, three steps with the cosine schedule."""
    from sparse_fine_tuning_amd.stack import MoEStack, cosine_lr
    dims = (200, 256, 8, 2, 96)
    T, H, E, K, I = dims
    L, steps, peak = 3, 3, 2e-4
    say(f"bf16 stack L={L} dims={dims}")
    R = O.Rounding(O.BF16, O.CONTRACT)
    layers = make_layers(L, dims, 0, bf16=True)
    shape = O.Shape(*dims)
    k = O.select_count(shape.N, 5, 1000)
    stk = MoEStack(L, *dims, act=capi.BF16, device=DEV)
    ref = []
    for l, lay in enumerate(layers):
        idx = synth.random_mask(shape.N, k, 50 + l)
        stk.load_layer(l, lay["W_gu"], lay["W_d"], lay["Wr"])
        stk.layers[l].set_active(torch.from_numpy(idx.view(np.int32)).to(DEV), capi.BF16)
        ref.append(dict(lay, idx=idx, m=np.zeros(k), v=np.zeros(k), mr=np.zeros_like(lay["Wr"]),
                        vr=np.zeros_like(lay["Wr"])))
    t_ref = 0
    for step in range(steps):
        X = synth.to_bf16_values(synth.normal((T, H), 1.0, 100 + step))
        tgt = synth.to_bf16_values(synth.normal((T, H), 1.0, 10000 + step))
        lr = cosine_lr(step, steps, peak)
        assert lr == O.cosine_lr(step, steps, peak)
        stk.set_batch(X, tgt)
        stk.train_step(lr)
        out = O.stack_train_step(X, tgt, ref, K, t_ref, lr, 0.9, 0.999, 1e-8, R)
        ref, t_ref = out["layers"], out["t"]
        torch.cuda.synchronize()
        assert abs(float(stk.loss.item()) - out["loss"]) <= TOL_BF16 * out["loss"], step
        # the last output of the stack
        assert rel(npf(stk.Xs[-1]), out["fwd"]["Xs"][-1]) <= TOL_BF16
        # the output gradient of layer 0, after the residual adds of the others
        assert rel(npf(stk.G[(L - 1) % 2]), out["bwd"]["dYs"][0]) <= TOL_BF16
        for l in range(L):
            assert rel(npf(stk.layers[l].dW), out["g"][l]) <= TOL_BF16, (step, l)
    assert stk.t == t_ref == steps
    for l in range(L):
        lay, r = stk.layers[l], ref[l]
        flat = np.concatenate([r["W_gu"].ravel(), r["W_d"].ravel()])
        assert rel(npf(lay.W), flat) <= TOL_BF16, l
        for got, want in ((lay.m, r["m"]), (lay.v, r["v"]), (lay.Wr, r["Wr"]), (lay.mr, r["mr"]),
                          (lay.vr, r["vr"])):
            assert rel(npf(got), want) <= TOL_BF16, l
        # weights outside the list are untouched, bit for bit
        w0 = np.concatenate([layers[l]["W_gu"].ravel(), layers[l]["W_d"].ravel()])
        off = np.ones(shape.N, bool)
        off[r["idx"].astype(np.int64)] = False
        assert np.array_equal(npf(lay.W)[off], w0[off])


def test_fp32_stack_importance_and_rigl(capi):
    """Tiny fp32 stack: every layer's dense gradient from one backward, its
    own top-5% selection, and a RigL pass at 30%."""
    from sparse_fine_tuning_amd.stack import MoEStack
    dims = (128, 64, 8, 2, 32)
    T, H, E, K, I = dims
    L = 3
    say(f"fp32 stack scan L={L} dims={dims}")
    R = O.Rounding(O.F32, O.CONTRACT)
    layers = make_layers(L, dims, 7, bf16=False)
    shape = O.Shape(*dims)
    k = O.select_count(shape.N, 5, 100)
    r = O.select_count(k, 3, 10)
    X = synth.normal((T, H), 1.0, 100)
    tgt = synth.normal((T, H), 1.0, 10000)
    stk = MoEStack(L, *dims, act=capi.F32, device=DEV)
    for l, lay in enumerate(layers):
        stk.load_layer(l, lay["W_gu"], lay["W_d"], lay["Wr"])
    stk.set_batch(X, tgt)
    grads = {}
    stk.forward()
    stk.backward(select=lambda l, g: grads.__setitem__(l, g.clone()))
    sc = O.stack_scan_grads(X, tgt, layers, K, R)
    for l in range(L):
        assert rel(npf(grads[l]), sc["grads"][l]) <= TOL_F32, l
    # each layer's own selection
    stk.importance(k)
    sel_ref = [O.importance_topk(sc["grads"][l], k) for l in range(L)]
    for l in range(L):
        sel = npu32(stk.layers[l].idx)
        assert sel.size == k and np.all(np.diff(sel.astype(np.int64)) > 0)
        assert k - np.intersect1d(sel, sel_ref[l]).size <= 2, l
    # identical gradients give identical selections
    from sparse_fine_tuning_amd.layer import topk
    for l in range(L):
        same = npu32(topk(torch.from_numpy(sc["grads"][l].astype(np.float32)).to(DEV), k))
        assert np.array_equal(same, sel_ref[l]), l
    # RigL from the oracle's selection, on the GPU's own gradients
    for l in range(L):
        stk.layers[l].set_active(torch.from_numpy(sel_ref[l].view(np.int32)).to(DEV), capi.F32)
    stats = stk.rigl(r).cpu().numpy()
    for l in range(L):
        flat = np.concatenate([layers[l]["W_gu"].ravel(), layers[l]["W_d"].ravel()]).astype(np.float64)
        want = O.rigl_reselect(sc["grads"][l], flat, sel_ref[l], np.zeros(k), np.zeros(k), k, r)
        new = npu32(stk.layers[l].idx)
        old = set(sel_ref[l].tolist())
        assert new.size == k and np.all(np.diff(new.astype(np.int64)) > 0)
        assert stats[l, 0] == r and stats[l, 1] == r
        assert len(old - set(new.tolist())) == r
        assert k - np.intersect1d(new, want["S_new"]).size <= 2, l
        # kept entries carry their moments (here zero), grown ones start at zero
        assert not np.any(npf(stk.layers[l].m)) and not np.any(npf(stk.layers[l].v))


# --------------------------------------------------------------------------
# the 48-layer Qwen3-shaped stack at its full size
# --------------------------------------------------------------------------
@pytest.mark.slow
def test_qwen3_stack_48_layers_full_size(capi):
    """48 layers of T=4096, H=2048, E=128, K=8, I=768 (bf16; device-drawn
    N(0, 0.02) weights and N(0, 1) batches from the stacked workload's
    seeds), importance at step 0, two steps, RigL at step 2 then a step.
    Checked: k ascending entries per layer, the RigL counts, finite losses,
    the shared step count, and every weight that was never listed
    bit-identical to its initial value."""
    from sparse_fine_tuning_amd.stack import MoEStack, cosine_lr
    dims = (4096, 2048, 128, 8, 768)
    T, H, E, K, I = dims
    L = 48
    say("qwen3 stack 48 layers: init")
    stk = MoEStack(L, *dims, act=capi.BF16, device=DEV)
    N = stk.shape.N
    k = (N * 5) // 1000
    r = (k * 3) // 10
    ngu = E * 2 * I * H

    def init_layer(l):
        g = torch.Generator(device=DEV)
        lay = stk.layers[l]
        g.manual_seed(1000 * (l + 1) + 1)
        lay.W[:ngu].copy_(torch.randn(ngu, generator=g, device=DEV) * 0.02)
        g.manual_seed(1000 * (l + 1) + 2)
        lay.W[ngu:].copy_(torch.randn(N - ngu, generator=g, device=DEV) * 0.02)
        g.manual_seed(1000 * (l + 1) + 3)
        lay.Wr.copy_(torch.randn(E, H, generator=g, device=DEV) * 0.02)

    for l in range(L):
        init_layer(l)

    def batch(t):
        g = torch.Generator(device=DEV)
        g.manual_seed(100 + t)
        X = torch.randn(T, H, generator=g, device=DEV)
        g.manual_seed(10000 + t)
        return X, torch.randn(T, H, generator=g, device=DEV)

    losses = []
    for t in range(3):
        stk.set_batch(*batch(t))
        if t == 0:
            say("importance")
            stk.importance(k)
        if t == 2:
            say("rigl")
            before = [lay.idx.to(torch.int64) for lay in stk.layers]
            stats = stk.rigl(r).cpu().numpy()
            assert np.all(stats[:, 0] == r) and np.all(stats[:, 1] == r)
            assert np.all(stats[:, 2] <= k)
        say(f"step {t}")
        stk.train_step(cosine_lr(t, 180, 2e-4))
        losses.append(float(stk.loss.item()))
    assert stk.t == 3 and stk.skipped == 0
    assert all(np.isfinite(losses))
    # per layer: the list, and weights outside it untouched
    rng = np.random.default_rng(1)
    probe = torch.from_numpy(np.unique(rng.integers(0, N, 200000)).astype(np.int64)).to(DEV)
    for l in range(L):
        idx = stk.layers[l].idx.to(torch.int64) & 0xFFFFFFFF
        assert idx.numel() == k and bool(torch.all(idx[1:] > idx[:-1]))
        W_now = stk.layers[l].W[probe].clone()
        init_layer(l)  # regenerate the initial weights in place of the trained ones
        W_init = stk.layers[l].W[probe]
        # trained at some step: listed before or after the reselection
        listed = torch.isin(probe, idx) | torch.isin(probe, before[l])
        assert torch.equal(W_now[~listed], W_init[~listed]), l
        assert bool((W_now[listed] != W_init[listed]).any()), l
        # RigL replaced r of the k entries
        assert int((~torch.isin(before[l], idx)).sum()) == r, l


# --------------------------------------------------------------------------
# trainer-loop features: frozen lower layers, expert load, the stack-wide
# NaN skip, and the bookkeeping merges
# --------------------------------------------------------------------------
def test_partial_stack_trains_upper_layers_only(capi):
    """Four bf16 layers with the two lowest frozen (the README's TRAIN_FROM):
    losses, the trained layers' gradients, weights, routers and moments
    against the oracle's stack step with the same train_from, and the frozen
    layers bit-identical to their initial weights and routers."""
    from sparse_fine_tuning_amd.stack import MoEStack, cosine_lr
    dims = (200, 256, 8, 2, 96)
    T, H, E, K, I = dims
    L, F, steps, peak = 4, 2, 2, 2e-4
    say(f"partial stack L={L} train_from={F} dims={dims}")
    R = O.Rounding(O.BF16, O.CONTRACT)
    layers = make_layers(L, dims, 11, bf16=True)
    shape = O.Shape(*dims)
    k = O.select_count(shape.N, 5, 1000)
    stk = MoEStack(L, *dims, act=capi.BF16, device=DEV, train_from=F)
    ref = []
    for l, lay in enumerate(layers):
        stk.load_layer(l, lay["W_gu"], lay["W_d"], lay["Wr"])
        if l < F:
            assert stk.layers[l].mr is None and stk.layers[l].idx is None
            ref.append(dict(lay))
            continue
        idx = synth.random_mask(shape.N, k, 70 + l)
        stk.layers[l].set_active(torch.from_numpy(idx.view(np.int32)).to(DEV), capi.BF16)
        ref.append(dict(lay, idx=idx, m=np.zeros(k), v=np.zeros(k), mr=np.zeros_like(lay["Wr"]),
                        vr=np.zeros_like(lay["Wr"])))
    t_ref = 0
    for step in range(steps):
        X = synth.to_bf16_values(synth.normal((T, H), 1.0, 120 + step))
        tgt = synth.to_bf16_values(synth.normal((T, H), 1.0, 12000 + step))
        lr = cosine_lr(step, steps, peak)
        stk.set_batch(X, tgt)
        stk.train_step(lr)
        out = O.stack_train_step(X, tgt, ref, K, t_ref, lr, 0.9, 0.999, 1e-8, R, train_from=F)
        ref, t_ref = out["layers"], out["t"]
        torch.cuda.synchronize()
        assert abs(float(stk.loss.item()) - out["loss"]) <= TOL_BF16 * out["loss"], step
        for l in range(F, L):
            assert rel(npf(stk.layers[l].dW), out["g"][l]) <= TOL_BF16, (step, l)
    assert stk.t == t_ref == steps
    for l in range(L):
        lay, r = stk.layers[l], ref[l]
        w0 = np.concatenate([layers[l]["W_gu"].ravel(), layers[l]["W_d"].ravel()])
        if l < F:
            assert np.array_equal(npf(lay.W), w0)
            assert np.array_equal(npf(lay.Wr), layers[l]["Wr"].astype(np.float32).astype(np.float64))
            continue
        flat = np.concatenate([r["W_gu"].ravel(), r["W_d"].ravel()])
        assert rel(npf(lay.W), flat) <= TOL_BF16, l
        for got, want in ((lay.m, r["m"]), (lay.v, r["v"]), (lay.Wr, r["Wr"]), (lay.mr, r["mr"]),
                          (lay.vr, r["vr"])):
            assert rel(npf(got), want) <= TOL_BF16, l


def test_expert_load_equals_the_oracle_grouping(capi):
    """expert_load() (the differences of each layer's expert offsets, a HIP
    kernel) against the oracle's group_by_expert counts of the same routing."""
    from sparse_fine_tuning_amd.stack import MoEStack
    dims = (200, 256, 8, 2, 96)
    T, H, E, K, I = dims
    L = 3
    say("expert load")
    layers = make_layers(L, dims, 13, bf16=True)
    stk = MoEStack(L, *dims, act=capi.BF16, device=DEV, train_from=1)
    for l, lay in enumerate(layers):
        stk.load_layer(l, lay["W_gu"], lay["W_d"], lay["Wr"])
    X = synth.to_bf16_values(synth.normal((T, H), 1.0, 130))
    stk.set_batch(X, X)
    stk.forward()
    load = stk.expert_load().cpu().numpy()
    assert load.shape == (L, E)
    for l in range(L):
        ids = stk.layers[l].st["topk_ids"].cpu().numpy()
        counts, _, _ = O.group_by_expert(ids, E)
        assert np.array_equal(load[l], counts), l
        assert load[l].sum() == T * K


def test_stack_nan_step_skips_every_layer(capi):
    """A non-finite target poisons the loss: no layer's weights, router or
    moments change, the step count stays and the skip is counted; the next
    finite step trains."""
    from sparse_fine_tuning_amd.stack import MoEStack
    dims = (200, 256, 8, 2, 96)
    T, H, E, K, I = dims
    L = 3
    say("stack NaN skip")
    layers = make_layers(L, dims, 17, bf16=True)
    shape = O.Shape(*dims)
    k = O.select_count(shape.N, 5, 1000)
    stk = MoEStack(L, *dims, act=capi.BF16, device=DEV)
    for l, lay in enumerate(layers):
        stk.load_layer(l, lay["W_gu"], lay["W_d"], lay["Wr"])
        stk.layers[l].set_active(torch.from_numpy(synth.random_mask(shape.N, k, 80 + l)
                                                  .view(np.int32)).to(DEV), capi.BF16)
        stk.layers[l].m.fill_(0.5)
        stk.layers[l].v.fill_(0.25)
    X = synth.to_bf16_values(synth.normal((T, H), 1.0, 140))
    tgt = synth.to_bf16_values(synth.normal((T, H), 1.0, 141))
    tgt[3, 5] = np.nan
    before = [(lay.W.clone(), lay.Wr.clone()) for lay in stk.layers]
    stk.set_batch(X, tgt)
    stk.train_step(1e-3)
    torch.cuda.synchronize()
    assert stk.skipped == 1 and stk.t == 0
    for lay, (W0, Wr0) in zip(stk.layers, before):
        assert torch.equal(lay.W.view(torch.int16), W0.view(torch.int16))
        assert torch.equal(lay.Wr, Wr0)
        assert bool((lay.m == 0.5).all()) and bool((lay.v == 0.25).all())
    tgt[3, 5] = 0.0
    stk.set_batch(X, tgt)
    stk.train_step(1e-3)
    torch.cuda.synchronize()
    assert stk.skipped == 1 and stk.t == 1
    assert not torch.equal(stk.layers[0].Wr, before[0][1])


@pytest.mark.parametrize("na,nb,overlap", [(0, 0, 0), (0, 1000, 0), (5000, 0, 0), (3000, 7000, 0.3),
                                           (100000, 90000, 0.5), (2048 * 3, 5, 1.0),
                                           (10, 300000, 0.0)])
def test_sorted_union_and_adjacent_diff(capi, na, nb, overlap):
    """usaf_sorted_union against numpy's union of two ascending lists (with
    shared entries, empty sides, a list far denser than the other); and
    usaf_adjacent_diff against numpy's diff."""
    say(f"sorted union na={na} nb={nb} overlap={overlap}")
    rng = np.random.default_rng(na + 7 * nb)
    a = np.sort(rng.choice(4 * (na + nb) + 10, na, replace=False)).astype(np.uint32)
    shared = rng.choice(a, int(overlap * min(na, nb)), replace=False) if na and nb else np.zeros(0, np.uint32)
    rest = np.setdiff1d(rng.choice(4 * (na + nb) + 10, 2 * nb + 10, replace=False).astype(np.uint32), a)
    b = np.sort(np.concatenate([shared, rest[: nb - shared.size]])).astype(np.uint32)
    want = np.union1d(a, b).astype(np.uint32)
    dev = lambda x: torch.from_numpy(x.view(np.int32).copy()).to(DEV)
    out = torch.full((max(na + b.size, 1),), -1, dtype=torch.int32, device=DEV)
    n_out = torch.zeros(1, dtype=torch.int64, device=DEV)
    ws = torch.empty(capi.workspace_size(capi.WS_UNION, None, na + b.size), dtype=torch.uint8,
                     device=DEV)
    capi.sorted_union(dev(a) if na else None, na, dev(b) if b.size else None, b.size, out, n_out, ws)
    torch.cuda.synchronize()
    n = int(n_out.item())
    assert n == want.size
    assert np.array_equal(npu32(out[:n]), want)
    if na > 1:
        offs = dev(np.sort(rng.integers(0, 1 << 20, na)).astype(np.int32).view(np.uint32))
        diff = torch.empty(na - 1, dtype=torch.int32, device=DEV)
        capi.adjacent_diff(offs, na - 1, diff)
        torch.cuda.synchronize()
        assert np.array_equal(diff.cpu().numpy(), np.diff(offs.cpu().numpy()))


def test_partial_stack_with_4bit_frozen_layers(capi):
    """Frozen layers kept as affine 4-bit codes (dequantised as their forward
    loads them) train the upper layers exactly as frozen layers holding the
    resident dequantised copy of the same codes: losses and every trained
    tensor bit-identical over two steps."""
    from sparse_fine_tuning_amd.stack import MoEStack
    dims = (200, 256, 8, 2, 128)
    T, H, E, K, I = dims
    L, F, group = 3, 2, 64
    say(f"partial stack, 4-bit frozen layers, dims={dims}")
    layers = make_layers(L, dims, 19, bf16=True)
    shape = O.Shape(*dims)
    k = O.select_count(shape.N, 5, 1000)
    codes = []
    for l in range(F):
        qg, sg, zg = synth.quantize_affine_int4(layers[l]["W_gu"].reshape(E * 2 * I, H), group)
        qd, sd, zd = synth.quantize_affine_int4(layers[l]["W_d"].reshape(E * H, I), group)
        codes.append((qg, sg, zg, qd, sd, zd))
    stacks = []
    for q4 in (False, True):
        stk = MoEStack(L, *dims, act=capi.BF16, device=DEV, train_from=F)
        for l, lay in enumerate(layers):
            if l < F:
                if q4:
                    stk.load_layer_q4(l, codes[l], group, lay["Wr"])
                else:  # the resident copy of the same codes
                    W_gu = O.dequant_affine(*codes[l][:3], group).reshape(E, 2 * I, H)
                    W_d = O.dequant_affine(*codes[l][3:], group).reshape(E, H, I)
                    stk.load_layer(l, W_gu, W_d, lay["Wr"])
            else:
                stk.load_layer(l, lay["W_gu"], lay["W_d"], lay["Wr"])
                stk.layers[l].set_active(torch.from_numpy(synth.random_mask(shape.N, k, 90 + l)
                                                          .view(np.int32)).to(DEV), capi.BF16)
        stacks.append(stk)
    for step in range(2):
        X = synth.to_bf16_values(synth.normal((T, H), 1.0, 150 + step))
        tgt = synth.to_bf16_values(synth.normal((T, H), 1.0, 15000 + step))
        for stk in stacks:
            stk.set_batch(X, tgt)
            stk.train_step(1e-3)
        torch.cuda.synchronize()
        assert float(stacks[0].loss.item()) == float(stacks[1].loss.item())
    a, b = stacks
    assert b.layers[0].W is None and a.t == b.t == 2
    for l in range(F, L):
        la, lb = a.layers[l], b.layers[l]
        assert torch.equal(la.W.view(torch.int16), lb.W.view(torch.int16))
        for x, y in ((la.m, lb.m), (la.v, lb.v), (la.Wr, lb.Wr), (la.mr, lb.mr), (la.vr, lb.vr)):
            assert torch.equal(x, y)

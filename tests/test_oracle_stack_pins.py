"""Pins of the oracle's stacked-layer functions (CPU only), against things other
than the oracle itself: torch float64 autograd through a token-by-token
stack, central finite differences of the stack loss, the reduction of a
one-layer stack to the single-layer step, the closed form of the cosine
schedule, and the all-layers NaN rule."""
import numpy as np
import torch

import usaf_synth as synth
from oracle import usaf_oracle as O

EX = O.Rounding(O.F32, O.EXACT)
C32 = O.Rounding(O.F32, O.CONTRACT)


def tiny_stack(L=3, T=24, H=16, E=6, K=2, I=8, seed=500):
    """L layers with weights 10x the workload's scale (so the nonlinearity
    matters), a fresh input and target."""
    layers = []
    for l in range(L):
        d = synth.moe_layer(T, H, E, K, I, bf16=False, seeds=tuple(seed + 10 * l + i for i in range(5)))
        layers.append(dict(W_gu=d["W_gu"] * 10, W_d=d["W_d"] * 10, Wr=d["Wr"] * 10))
    X0 = synth.normal((T, H), 1.0, seed + 1000)
    tgt = synth.normal((T, H), 1.0, seed + 1001)
    return layers, X0, tgt


def autograd_stack(layers, X0, tgt, K):
    """torch float64 autograd: per token, top-K routing on the logits, softmax
    over the K, SwiGLU experts; X_{l+1} = X_l + Y_l; MSE of X_L."""
    params = [dict(W_gu=torch.from_numpy(l["W_gu"]).double().requires_grad_(),
                   W_d=torch.from_numpy(l["W_d"]).double().requires_grad_(),
                   Wr=torch.from_numpy(l["Wr"]).double().requires_grad_()) for l in layers]
    X = torch.from_numpy(X0).double().requires_grad_()
    h = X
    for p in params:
        I = p["W_d"].shape[2]
        rows = []
        for t in range(h.shape[0]):
            lg = p["Wr"] @ h[t]
            top = torch.topk(lg.detach(), K).indices
            wts = torch.softmax(lg[top], 0)
            acc = 0
            for j in range(K):
                e = int(top[j])
                gu = p["W_gu"][e] @ h[t]
                acc = acc + wts[j] * (p["W_d"][e] @ (torch.nn.functional.silu(gu[:I]) * gu[I:]))
            rows.append(acc)
        h = h + torch.stack(rows)
    loss = torch.nn.functional.mse_loss(h, torch.from_numpy(tgt).double())
    loss.backward()
    return loss.item(), X.grad.numpy(), [{k: v.grad.numpy() for k, v in p.items()} for p in params]


def test_stack_backward_matches_autograd():
    K = 2
    layers, X0, tgt = tiny_stack()
    sc = O.stack_scan_grads(X0, tgt, layers, K, EX)
    loss, gX, gps = autograd_stack(layers, X0, tgt, K)
    assert abs(sc["loss"] - loss) <= 1e-13 * max(1.0, loss)
    scale = np.abs(gX).max()
    assert np.abs(sc["bwd"]["G0"] - gX).max() <= 1e-12 * scale
    for l, lay in enumerate(layers):
        shape = O.Shape(X0.shape[0], X0.shape[1], lay["W_gu"].shape[0], K, lay["W_d"].shape[2])
        Wgu_g, Wd_g = O.unflatten(sc["grads"][l], shape)
        for got, want in ((Wgu_g, gps[l]["W_gu"]), (Wd_g, gps[l]["W_d"]),
                          (sc["bwd"]["bws"][l]["dWr"], gps[l]["Wr"])):
            assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max(), l


def test_stack_finite_differences():
    K = 2
    layers, X0, tgt = tiny_stack(L=2, seed=600)
    sc = O.stack_scan_grads(X0, tgt, layers, K, EX)
    ids0 = [fw["topk_ids"] for fw in sc["fwd"]["fws"]]
    rng = np.random.default_rng(9)

    def loss_of(lays, x0):
        fwd = O.stack_forward(x0, lays, K, EX)
        for fw, ids in zip(fwd["fws"], ids0):
            assert np.array_equal(fw["topk_ids"], ids), "routing changed under perturbation"
        return O.mse_loss_grad(fwd["Xs"][-1], tgt, EX)[0]

    for l in range(2):
        shape = O.Shape(X0.shape[0], X0.shape[1], layers[l]["W_gu"].shape[0], K, layers[l]["W_d"].shape[2])
        Wgu_g, Wd_g = O.unflatten(sc["grads"][l], shape)
        for name, grad in (("W_gu", Wgu_g), ("W_d", Wd_g), ("Wr", sc["bwd"]["bws"][l]["dWr"])):
            base = layers[l][name].astype(np.float64)
            scale = np.abs(grad).max()
            for _ in range(8):
                pos = tuple(rng.integers(0, n) for n in base.shape)
                h = 1e-5 * max(1.0, abs(base[pos]))
                vals = []
                for sgn in (1, -1):
                    lays = [dict(x) for x in layers]
                    w = base.copy()
                    w[pos] += sgn * h
                    lays[l] = dict(lays[l], **{name: w})
                    vals.append(loss_of(lays, X0))
                fd = (vals[0] - vals[1]) / (2 * h)
                assert abs(fd - grad[pos]) <= 1e-6 * scale, (l, name, pos, fd, grad[pos])
    G0 = sc["bwd"]["G0"]
    for _ in range(8):
        pos = tuple(rng.integers(0, n) for n in X0.shape)
        h = 1e-5 * max(1.0, abs(X0[pos]))
        up, dn = X0.astype(np.float64).copy(), X0.astype(np.float64).copy()
        up[pos] += h
        dn[pos] -= h
        fd = (loss_of(layers, up) - loss_of(layers, dn)) / (2 * h)
        assert abs(fd - G0[pos]) <= 1e-6 * np.abs(G0).max()


def test_one_layer_stack_is_the_layer_step_on_the_residual_target():
    """X_1 = X_0 + Y, so MSE(X_1, tgt) = MSE(Y, tgt - X_0): in exact mode the
    one-layer stack step equals the layer step on the shifted target."""
    K = 2
    layers, X0, tgt = tiny_stack(L=1, seed=700)
    lay = layers[0]
    shape = O.Shape(X0.shape[0], X0.shape[1], lay["W_gu"].shape[0], K, lay["W_d"].shape[2])
    k = O.select_count(shape.N, 5, 100)
    idx = synth.random_mask(shape.N, k, 7)
    st = dict(lay, idx=idx, m=np.zeros(k), v=np.zeros(k), mr=np.zeros_like(lay["Wr"]),
              vr=np.zeros_like(lay["Wr"]))
    out = O.stack_train_step(X0, tgt, [st], K, 0, 1e-3, 0.9, 0.999, 1e-8, EX)
    shifted = tgt.astype(np.float64) - X0.astype(np.float64)
    ref = O.train_step(X0, shifted, lay["Wr"], lay["W_gu"], lay["W_d"], K, idx, st["m"], st["v"],
                       st["mr"], st["vr"], 0, 1e-3, 0.9, 0.999, 1e-8, EX)
    assert abs(out["loss"] - ref["loss"]) <= 1e-14 * ref["loss"]
    assert out["t"] == ref["t"] == 1
    new = out["layers"][0]
    flat = np.concatenate([new["W_gu"].ravel(), new["W_d"].ravel()])
    assert np.abs(flat - ref["W_flat"]).max() <= 1e-15
    for key in ("m", "v", "Wr", "mr", "vr"):
        assert np.abs(new[key] - ref[key]).max() <= 1e-15 * max(1.0, np.abs(ref[key]).max()), key
    # the input gradient adds the residual path to the layer's own dX
    G0 = out["bwd"]["G0"]
    assert np.abs(G0 - (ref["dY"] + ref["bw"]["dX"])).max() <= 1e-15 * np.abs(G0).max()


def test_zero_down_projections_pass_the_gradient_through():
    """With every W_d = 0 each layer outputs 0, so X_L = X_0, and every
    layer's input gradient vanishes, so G_0 = G_L exactly (contract mode)."""
    K = 2
    layers, X0, tgt = tiny_stack(L=3, seed=800)
    for lay in layers:
        lay["W_d"] = np.zeros_like(lay["W_d"])
    X0c = C32.act(X0)
    fwd = O.stack_forward(X0c, layers, K, C32)
    assert np.array_equal(fwd["Xs"][-1], X0c)
    loss, GL = O.mse_loss_grad(fwd["Xs"][-1], tgt, C32)
    bwd = O.stack_backward(fwd, layers, GL, C32)
    assert np.array_equal(bwd["G0"], GL)


def test_stack_nan_skips_every_layer():
    K = 2
    layers, X0, tgt = tiny_stack(L=2, seed=900)
    sts = []
    for lay in layers:
        shape = O.Shape(X0.shape[0], X0.shape[1], lay["W_gu"].shape[0], K, lay["W_d"].shape[2])
        k = O.select_count(shape.N, 5, 100)
        sts.append(dict(lay, idx=synth.random_mask(shape.N, k, 3), m=np.zeros(k), v=np.zeros(k),
                        mr=np.zeros_like(lay["Wr"]), vr=np.zeros_like(lay["Wr"])))
    sts[1]["W_d"] = sts[1]["W_d"].copy()
    sts[1]["W_d"][0, 0, 0] = np.inf
    out = O.stack_train_step(X0, tgt, sts, K, 4, 1e-3, 0.9, 0.999, 1e-8, C32)
    assert out["skipped"] and out["t"] == 4
    for new, old in zip(out["layers"], sts):
        for key in ("W_gu", "W_d", "Wr", "m", "v", "mr", "vr"):
            assert np.array_equal(new[key], old[key]), key


def test_residual_add_rounds_once():
    a = np.array([1.0, 1.0, 3.0, -2.0 ** -7], dtype=np.float64)
    b = np.array([2.0 ** -8, 3 * 2.0 ** -9, 2.0 ** -20, 2.0 ** -7])
    R = O.Rounding(O.BF16, O.CONTRACT)
    got = O.residual_add(a, b, R)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 (even: 1); 1 + 3*2^-9 rounds up
    assert got.tolist() == [1.0, 1.0 + 2.0 ** -7, 3.0, 0.0]


def test_cosine_lr_closed_form():
    peak, total = 2e-4, 180
    assert O.cosine_lr(0, total, peak) == peak
    assert abs(O.cosine_lr(total // 2, total, peak) - peak / 2) <= 1e-20
    assert abs(O.cosine_lr(total, total, peak)) <= 1e-20
    for t in range(total):
        assert abs(O.cosine_lr(t, total, peak) + O.cosine_lr(total - t, total, peak) - peak) <= 1e-19
        assert O.cosine_lr(t + 1, total, peak) < O.cosine_lr(t, total, peak)


def test_frozen_lower_layers_train_as_in_the_full_stack():
    """With the layers below train_from frozen, each trained layer gets the
    very update it gets when every layer trains (its gradients come from the
    layers above it only), the frozen layers are unchanged, bit for bit, and
    need no list or moments."""
    R = O.Rounding(O.BF16, O.CONTRACT)
    dims = (24, 16, 4, 2, 8)
    T, H, E, K, I = dims
    layers = []
    for l in range(4):
        d = synth.moe_layer(*dims, bf16=True, seeds=tuple(500 + 10 * l + j for j in range(5)))
        N = 3 * E * H * I
        k = O.select_count(N, 5, 100)
        layers.append(dict(W_gu=d["W_gu"] * 10, W_d=d["W_d"] * 10, Wr=d["Wr"] * 10,
                           idx=synth.random_mask(N, k, 600 + l), m=np.zeros(k), v=np.zeros(k),
                           mr=np.zeros((E, H)), vr=np.zeros((E, H))))
    X0 = synth.to_bf16_values(synth.normal((T, H), 1.0, 700))
    tgt = synth.to_bf16_values(synth.normal((T, H), 1.0, 701))
    full = O.stack_train_step(X0, tgt, layers, K, 0, 1e-3, 0.9, 0.999, 1e-8, R)
    part = O.stack_train_step(X0, tgt, layers, K, 0, 1e-3, 0.9, 0.999, 1e-8, R, train_from=2)
    assert part["t"] == full["t"] == 1
    for l in range(4):
        for key in ("W_gu", "W_d", "Wr", "m", "v", "mr", "vr"):
            want = (full if l >= 2 else dict(layers=layers))["layers"][l][key]
            assert np.array_equal(part["layers"][l][key], want), (l, key)
    # frozen layers need no list and no moments
    bare = [dict(W_gu=lay["W_gu"], W_d=lay["W_d"], Wr=lay["Wr"]) for lay in layers[:2]] + layers[2:]
    out = O.stack_train_step(X0, tgt, bare, K, 0, 1e-3, 0.9, 0.999, 1e-8, R, train_from=2)
    for l in range(2, 4):
        assert np.array_equal(out["layers"][l]["W_gu"], full["layers"][l]["W_gu"])

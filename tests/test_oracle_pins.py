"""Pins of the CPU oracle against things other than itself.

Each test checks one oracle function against a closed form, a brute force on a
tiny input, a library routine that reaches the same result by another route
(torch autograd, torch.optim.Adam, torch's bf16 conversion), finite
differences, or a page-printed number.  Chosen so that a dropped term, a wrong
sign or index, or a transposed operand in the oracle fails at least one.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import usaf_synth as synth
from oracle import usaf_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EX = O.Rounding(O.F32, O.EXACT)
C32 = O.Rounding(O.F32, O.CONTRACT)
CB16 = O.Rounding(O.BF16, O.CONTRACT)


def tiny_layer(T=32, H=16, E=6, K=2, I=8, seed=100, bf16=False):
    d = synth.moe_layer(T, H, E, K, I, bf16=bf16, seeds=tuple(seed + i for i in range(5)))
    # larger weights than the workload's 0.02 so the nonlinearity matters
    d["W_gu"] = d["W_gu"] * 10
    d["W_d"] = d["W_d"] * 10
    d["Wr"] = d["Wr"] * 10
    return d


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------
def test_bf16_rne_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    # add exact ties (low 16 bits = 0x8000) and near-ties, subnormals, extremes
    ties = (rng.integers(0, 2 ** 16, size=5000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    special = np.array([0, 0x80000000, 0x00000001, 0x00008000, 0x00018000, 0x7F7FFFFF,
                        0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000,
                        0x3F808000, 0x3F818000], dtype=np.uint32)
    allb = np.concatenate([bits, ties, special])
    x = allb.view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    got = O.bf16_rne(x).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_rne_fp64_against_brute_force_nearest():
    # every finite non-negative bf16 value, ascending
    pos = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    grid = pos.view(np.float32).astype(np.float64)
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        (grid[1:200] + grid[:199]) / 2.0,  # exact midpoints incl. subnormals
                        (grid[30000:30200] + grid[30001:30201]) / 2.0])
    got = O.bf16_rne(x)
    ax = np.abs(x)
    hi = np.clip(np.searchsorted(grid, ax), 1, grid.size - 1)
    lo = hi - 1
    dlo, dhi = ax - grid[lo], grid[hi] - ax
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))  # even mantissa = even index
    want = np.where(pick_hi, grid[hi], grid[lo]) * np.sign(x)
    assert np.array_equal(got, want)
    assert np.isnan(O.bf16_rne(np.nan)) and O.bf16_rne(np.inf) == np.inf
    assert O.bf16_rne(3.5e38) == np.inf


# --------------------------------------------------------------------------
# a1 dequant
# --------------------------------------------------------------------------
def test_dequant_exhaustive_codes_and_scales():
    # scales: zero, subnormal fp16, normal, the fp16 max, negative
    scales = np.array([0.0, 5.96e-8, 6.1e-5, 1e-3, 0.0123, 0.5, 1.0, 3.14, 1000.0, 65504.0,
                       -0.02], dtype=np.float16)
    codes = np.arange(-8, 8)
    rows = scales.size
    q = np.tile(codes, (rows, 4))  # 64 columns per row = one group
    nib = (q & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    got = O.dequant_int4(packed, scales.view(np.uint16).reshape(rows, 1), group=64)
    prod = torch.from_numpy(q.astype(np.float32)) * torch.from_numpy(
        scales.astype(np.float32)).reshape(rows, 1)
    want = prod.to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)


def test_dequant_nibble_order_and_groups():
    # byte 0x9F holds element 0 = low nibble 0xF (-1), element 1 = high nibble 0x9 (-7)
    packed = np.full((1, 64), 0x9F, dtype=np.uint8)  # 128 columns = 2 groups
    sc = np.array([[2.0, -0.5]], dtype=np.float16).view(np.uint16)
    got = O.dequant_int4(packed, sc, group=64)
    assert got[0, 0] == -2.0 and got[0, 1] == -14.0
    assert got[0, 64] == 0.5 and got[0, 65] == 3.5


def pack_unsigned(codes):
    c = np.asarray(codes, np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def test_affine_dequant_with_zero_8_is_the_symmetric_format():
    """Offset-binary codes u = c + 8 with zero 8 give (u - 8) s = c s: the
    affine dequant must equal the symmetric int4 dequant (pinned above) with
    the same scale in both of its 64-wide halves."""
    rng = np.random.default_rng(31)
    rows, cols = 6, 256
    c = rng.integers(-8, 8, size=(rows, cols))
    sc = (10.0 ** rng.uniform(-6, 3, size=(rows, cols // 128)) * rng.choice([-1, 1], (rows, cols // 128))).astype(np.float16)
    nib = (c & 0xF).astype(np.uint8)
    sym = O.dequant_int4((nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8),
                         np.repeat(sc, 2, axis=1).view(np.uint16), group=64)
    zero = np.full(sc.shape, 8.0, np.float16)
    aff = O.dequant_affine(pack_unsigned(c + 8), sc.view(np.uint16), zero.view(np.uint16), group=128)
    assert np.array_equal(aff, sym)


def test_affine_dequant_exact_cases_by_hand():
    # zero 2.5, scale 2^-6: (q - 2.5) / 64 is exact in fp32 and in bf16
    q = np.tile(np.arange(16), (1, 8))  # 128 columns = one group
    got = O.dequant_affine(pack_unsigned(q), np.array([[2.0 ** -6]], np.float16).view(np.uint16),
                           np.array([[2.5]], np.float16).view(np.uint16))
    assert np.array_equal(got[0, :16], (np.arange(16) - 2.5) / 64.0)
    # q == zero gives exactly 0 whatever the scale
    got = O.dequant_affine(pack_unsigned(np.full((1, 128), 7)), np.array([[65504.0]], np.float16).view(np.uint16),
                           np.array([[7.0]], np.float16).view(np.uint16))
    assert np.all(got == 0.0)


def test_affine_dequant_rounds_in_fp32_first():
    """The reading's two fp32 roundings, worked by hand: q = 1, z = -2^-24,
    s = 1 + 2^-8.  In fp32, 1 + 2^-24 is a tie that rounds to 1; 1 * s = 1 + 2^-8
    is then a bf16 tie that rounds to even: 1.  Exact arithmetic would give
    1 + 2^-8 + 2^-24 + 2^-32, above the tie: 1 + 2^-7."""
    codes = np.ones((1, 128), np.uint8)
    got = O.dequant_affine(pack_unsigned(codes), np.array([[1 + 2.0 ** -8]], np.float16).view(np.uint16),
                           np.array([[-(2.0 ** -24)]], np.float16).view(np.uint16))
    assert np.all(got == 1.0)
    assert float(np.float16(-(2.0 ** -24))) == -(2.0 ** -24)  # the smallest fp16 subnormal


def test_affine_dequant_matches_torch_fp32_then_bf16():
    rng = np.random.default_rng(33)
    rows, cols = 16, 256
    q = rng.integers(0, 16, size=(rows, cols))
    sc = (10.0 ** rng.uniform(-7, 4, size=(rows, 2))).astype(np.float16)
    zr = rng.uniform(-2, 17, size=(rows, 2)).astype(np.float16)
    got = O.dequant_affine(pack_unsigned(q), sc.view(np.uint16), zr.view(np.uint16))
    qt = torch.from_numpy(q.astype(np.float32))
    st = torch.from_numpy(np.repeat(sc.astype(np.float32), 128, axis=1))
    zt = torch.from_numpy(np.repeat(zr.astype(np.float32), 128, axis=1))
    want = ((qt - zt) * st).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)


def test_affine_roundtrip_of_synthetic_quantizer():
    w = synth.normal((8, 256), 0.02, 9)
    q, s, z = synth.quantize_affine_int4(w, 128)
    back = O.dequant_affine(q, s, z, 128)
    scale = np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)
    assert np.all(np.abs(back - w) <= 0.55 * scale + 2.0 ** -8 * np.abs(w).max())


def test_dequant_roundtrip_of_synthetic_quantizer():
    w = synth.normal((8, 128), 0.02, 7)
    q, s = synth.quantize_int4_g64(w)
    back = O.dequant_int4(q, s)
    scale = np.repeat(s.view(np.float16).astype(np.float64), 64, axis=1)
    assert np.all(np.abs(back - w) <= 0.5 * scale * (1 + 1e-2) + 1e-12)


# --------------------------------------------------------------------------
# a2-a4 routing
# --------------------------------------------------------------------------
@pytest.mark.parametrize("E,K", [(8, 2), (6, 3), (5, 1), (4, 4)])
def test_route_topk_brute_force_subsets(E, K):
    rng = np.random.default_rng(E * 10 + K)
    T = 300
    logits = rng.integers(-3, 3, size=(T, E)).astype(np.float64) * 0.25  # tie-heavy
    logits[: T // 2] += rng.standard_normal((T // 2, E))
    ids, w = O.route_topk(logits, K, EX)
    for t in range(T):
        valid = []
        for sub in itertools.combinations(range(E), K):
            rest = [j for j in range(E) if j not in sub]
            ok = all(logits[t, i] > logits[t, j] or (logits[t, i] == logits[t, j] and i < j)
                     for i in sub for j in rest)
            if ok:
                valid.append(sub)
        assert len(valid) == 1
        order = sorted(valid[0], key=lambda i: (-logits[t, i], i))
        assert list(ids[t]) == order
        full = torch.softmax(torch.from_numpy(logits[t]), dim=0).numpy()
        ref = full[order] / full[order].sum()
        np.testing.assert_allclose(w[t], ref, rtol=1e-13, atol=1e-15)
        assert abs(w[t].sum() - 1.0) < 1e-12 and np.all(w[t] >= 0)


def test_route_topk_fp32_weights_sum_to_one():
    rng = np.random.default_rng(3)
    logits = O.f32_rne(rng.standard_normal((500, 16)))
    _, w = O.route_topk(logits, 4, C32)
    assert np.all(np.abs(w.sum(1) - 1.0) <= 4 * 2.0 ** -23)


def test_group_by_expert_brute_force():
    rng = np.random.default_rng(4)
    T, E, K = 200, 7, 3
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    counts, offsets, perm = O.group_by_expert(ids, E)
    assert sorted(perm.tolist()) == list(range(T * K))
    assert counts.sum() == T * K and offsets[0] == 0 and offsets[-1] == T * K
    for e in range(E):
        want = [s for s in range(T * K) if ids.reshape(-1)[s] == e]
        assert perm[offsets[e]:offsets[e + 1]].tolist() == want
        assert counts[e] == len(want)


def test_router_logits_fp32_and_bf16_weight():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((10, 12))
    Wr = rng.standard_normal((4, 12)) * 0.02
    lt = torch.from_numpy(X) @ torch.from_numpy(Wr).T
    np.testing.assert_allclose(O.router_logits(X, Wr, EX), lt.numpy(), rtol=1e-14, atol=1e-16)
    Wb = torch.from_numpy(Wr.astype(np.float32)).to(torch.bfloat16).to(torch.float64)
    lb = (torch.from_numpy(X) @ Wb.T).to(torch.float32).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.router_logits(X, Wr, CB16), lb)


# --------------------------------------------------------------------------
# a5-a6 forward
# --------------------------------------------------------------------------
def per_token_forward(d, K):
    """Token-by-token evaluation with torch: route one token, run each chosen
    expert on that token vector alone, add the weighted outputs."""
    X = torch.from_numpy(d["X"]).double()
    Wgu = torch.from_numpy(d["W_gu"]).double()
    Wd = torch.from_numpy(d["W_d"]).double()
    Wr = torch.from_numpy(d["Wr"]).double()
    I = Wd.shape[2]
    Y = torch.zeros_like(X)
    for t in range(X.shape[0]):
        lg = Wr @ X[t]
        p = torch.softmax(lg, 0)
        top = torch.topk(lg, K).indices
        wts = p[top] / p[top].sum()
        for j in range(K):
            e = int(top[j])
            h = Wgu[e] @ X[t]
            a = torch.nn.functional.silu(h[:I]) * h[I:]
            Y[t] += wts[j] * (Wd[e] @ a)
    return Y.numpy()


def test_forward_matches_per_token_evaluation():
    d = tiny_layer()
    fw = O.moe_forward(d["X"], d["Wr"], d["W_gu"], d["W_d"], 2, EX)
    np.testing.assert_allclose(fw["Y"], per_token_forward(d, 2), rtol=1e-12, atol=1e-14)


def test_single_expert_is_textbook_swiglu_mlp():
    d = tiny_layer(E=1, K=1)
    fw = O.moe_forward(d["X"], d["Wr"], d["W_gu"], d["W_d"], 1, EX)
    assert np.all(fw["topk_w"] == 1.0)
    X = torch.from_numpy(d["X"]).double()
    I = d["W_d"].shape[2]
    gate = torch.nn.functional.linear(X, torch.from_numpy(d["W_gu"][0, :I]).double())
    up = torch.nn.functional.linear(X, torch.from_numpy(d["W_gu"][0, I:]).double())
    Y = torch.nn.functional.linear(torch.nn.functional.silu(gate) * up,
                                   torch.from_numpy(d["W_d"][0]).double())
    np.testing.assert_allclose(fw["Y"], Y.numpy(), rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# a7-a13 gradients
# --------------------------------------------------------------------------
def test_mse_grad_matches_autograd():
    rng = np.random.default_rng(6)
    Y = rng.standard_normal((9, 7))
    tgt = rng.standard_normal((9, 7))
    loss, dY = O.mse_loss_grad(Y, tgt, EX)
    y = torch.from_numpy(Y).requires_grad_()
    L = torch.nn.functional.mse_loss(y, torch.from_numpy(tgt))
    L.backward()
    assert abs(loss - L.item()) < 1e-14
    np.testing.assert_allclose(dY, y.grad.numpy(), rtol=1e-13)


def autograd_grads(d, K):
    """torch float64 autograd through a token-by-token formulation."""
    X = torch.from_numpy(d["X"]).double().requires_grad_()
    Wgu = torch.from_numpy(d["W_gu"]).double().requires_grad_()
    Wd = torch.from_numpy(d["W_d"]).double().requires_grad_()
    Wr = torch.from_numpy(d["Wr"]).double().requires_grad_()
    tgt = torch.from_numpy(d["tgt"]).double()
    I = Wd.shape[2]
    rows = []
    for t in range(X.shape[0]):
        lg = Wr @ X[t]
        top = torch.topk(lg.detach(), K).indices
        wts = torch.softmax(lg[top], 0)
        acc = 0
        for j in range(K):
            e = int(top[j])
            h = Wgu[e] @ X[t]
            acc = acc + wts[j] * (Wd[e] @ (torch.nn.functional.silu(h[:I]) * h[I:]))
        rows.append(acc)
    Y = torch.stack(rows)
    L = torch.nn.functional.mse_loss(Y, tgt)
    L.backward()
    return dict(X=X.grad.numpy(), W_gu=Wgu.grad.numpy(), W_d=Wd.grad.numpy(),
                Wr=Wr.grad.numpy(), loss=L.item())


@pytest.mark.parametrize("E,K", [(6, 2), (4, 3), (1, 1)])
def test_backward_matches_autograd(E, K):
    d = tiny_layer(E=E, K=K, seed=200 + E)
    shape = O.Shape(32, 16, E, K, 8)
    sc = O.dense_scan(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, EX)
    ref = autograd_grads(d, K)
    assert abs(sc["loss"] - ref["loss"]) < 1e-13
    Wgu_g, Wd_g = O.unflatten(sc["g"], shape)
    for got, want in ((Wgu_g, ref["W_gu"]), (Wd_g, ref["W_d"]),
                      (sc["bw"]["dWr"], ref["Wr"]), (sc["bw"]["dX"], ref["X"])):
        scale = np.abs(want).max()
        assert np.abs(got - want).max() <= 1e-12 * scale


def test_backward_finite_differences():
    d = tiny_layer(seed=300)
    K = 2
    shape = O.Shape(32, 16, 6, K, 8)
    sc = O.dense_scan(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, EX)
    ids0 = sc["fw"]["topk_ids"]
    Wgu_g, Wd_g = O.unflatten(sc["g"], shape)
    rng = np.random.default_rng(8)

    def loss_of(dd):
        fw = O.moe_forward(dd["X"], dd["Wr"], dd["W_gu"], dd["W_d"], K, EX)
        assert np.array_equal(fw["topk_ids"], ids0), "routing changed under perturbation"
        return O.mse_loss_grad(fw["Y"], dd["tgt"], EX)[0]

    for name, grad in (("W_gu", Wgu_g), ("W_d", Wd_g), ("Wr", sc["bw"]["dWr"]),
                       ("X", sc["bw"]["dX"])):
        base = d[name].astype(np.float64)
        scale = np.abs(grad).max()
        for _ in range(12):
            pos = tuple(rng.integers(0, n) for n in base.shape)
            h = 1e-5 * max(1.0, abs(base[pos]))
            up = dict(d); dn = dict(d)
            up[name] = base.copy(); up[name][pos] += h
            dn[name] = base.copy(); dn[name][pos] -= h
            fd = (loss_of(up) - loss_of(dn)) / (2 * h)
            assert abs(fd - grad[pos]) <= 1e-6 * scale, (name, pos, fd, grad[pos])


def test_dlogits_sum_to_zero_per_token():
    d = tiny_layer(seed=400)
    sc = O.dense_scan(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], 2, EX)
    dl = sc["bw"]["dlogits"]
    assert np.abs(dl.sum(axis=1)).max() <= 1e-15 * max(1.0, np.abs(dl).max()) * 10
    assert np.count_nonzero(dl, axis=1).max() <= 2


def test_masked_at_full_density_equals_dense():
    d = tiny_layer(seed=500)
    shape = O.Shape(32, 16, 6, 2, 8)
    for R in (EX, C32):
        sc = O.dense_scan(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], 2, R)
        allidx = np.arange(shape.N)
        g = O.weight_grads_at(sc["fw"], sc["bw"], d["X"], sc["dY"], allidx, shape, R)
        np.testing.assert_allclose(g, sc["g"], rtol=1e-12, atol=1e-18)


def test_split_flat_matches_unravel():
    shape = O.Shape(4, 16, 3, 2, 8)
    f = np.arange(shape.N)
    tens, e, r, c = O.split_flat(f, shape)
    ngu = shape.n_gate_up
    e1, r1, c1 = np.unravel_index(f[:ngu], (3, 16, 16))
    e2, r2, c2 = np.unravel_index(f[ngu:] - ngu, (3, 16, 8))
    assert np.all(tens[:ngu] == 0) and np.all(tens[ngu:] == 1)
    assert np.array_equal(e, np.concatenate([e1, e2]))
    assert np.array_equal(r, np.concatenate([r1, r2]))
    assert np.array_equal(c, np.concatenate([c1, c2]))


def test_contract_close_to_exact():
    d = synth.moe_layer(64, 32, 4, 2, 16, bf16=True, seeds=(9, 10, 11, 12, 13))
    a = O.dense_scan(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], 2, EX)
    b = O.dense_scan(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], 2, CB16)
    assert np.array_equal(a["fw"]["topk_ids"], b["fw"]["topk_ids"])
    for x, y in ((a["fw"]["Y"], b["fw"]["Y"]), (a["g"], b["g"]), (a["bw"]["dX"], b["bw"]["dX"])):
        assert np.abs(x - y).max() <= 2e-2 * np.abs(x).max()


# --------------------------------------------------------------------------
# a12 Adam
# --------------------------------------------------------------------------
def test_adam_first_step_closed_form():
    rng = np.random.default_rng(9)
    g = rng.standard_normal(1000) * 10.0 ** rng.integers(-9, 0, 1000)
    w = rng.standard_normal(1000)
    lr, eps = 1e-3, 1e-8
    w1, m1, v1 = O.adam_update(w, g, np.zeros(1000), np.zeros(1000), 1, lr, 0.9, 0.999, eps,
                               O.F32, EX)
    np.testing.assert_allclose(w1 - w, -lr * g / (np.abs(g) + eps), rtol=1e-9, atol=1e-18)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-14)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-12)


def test_adam_matches_torch_optim_over_steps():
    rng = np.random.default_rng(10)
    n, lr, b1, b2, eps = 257, 1e-3, 0.9, 0.999, 1e-8
    w0 = rng.standard_normal(n)
    grads = [rng.standard_normal(n) * 1e-3 for _ in range(6)]
    p = torch.nn.Parameter(torch.from_numpy(w0.copy()))
    opt = torch.optim.Adam([p], lr=lr, betas=(b1, b2), eps=eps)
    w, m, v = w0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        w, m, v = O.adam_update(w, g, m, v, t, lr, b1, b2, eps, O.F32, EX)
    np.testing.assert_allclose(w, p.detach().numpy(), rtol=1e-12, atol=1e-15)


def test_adam_bf16_weight_rounding():
    w = O.bf16_rne(np.array([1.0, -0.5, 0.02]))
    g = np.array([1e-3, -2e-3, 0.0])
    w1, _, _ = O.adam_update(w, g, np.zeros(3), np.zeros(3), 1, 1e-3, 0.9, 0.999, 1e-8,
                             O.BF16, CB16)
    assert np.array_equal(w1, O.bf16_rne(w1))
    assert w1[2] == w[2]  # zero gradient, zero moments -> no change


# --------------------------------------------------------------------------
# a14 top-k, a15 RigL
# --------------------------------------------------------------------------
def brute_topk(g, k, exclude=()):
    ex = set(int(i) for i in exclude)
    cand = [i for i in range(len(g)) if i not in ex]
    mag = np.abs(np.asarray(g, dtype=np.float32))
    order = sorted(cand, key=lambda i: (-float(mag[i]), i))
    return np.array(sorted(order[:k]), dtype=np.uint32)


@pytest.mark.parametrize("N,k,levels", [(1000, 50, 0), (3000, 700, 3), (513, 513, 2),
                                        (400, 0, 0), (2000, 1, 1)])
def test_topk_brute_force(N, k, levels):
    rng = np.random.default_rng(N + k)
    g = rng.standard_normal(N).astype(np.float32)
    if levels:
        g = (rng.integers(0, levels, N) * 0.5 * np.sign(g)).astype(np.float32)
    got = O.importance_topk(g, k)
    assert np.array_equal(got, brute_topk(g, k))
    assert got.size == k and np.all(np.diff(got.astype(np.int64)) > 0)
    if 0 < k < N:
        mag = np.abs(g)
        sel = np.zeros(N, bool); sel[got] = True
        assert mag[sel].min() >= mag[~sel].max()


def test_topk_with_exclusion_brute_force():
    rng = np.random.default_rng(11)
    g = (rng.integers(0, 4, 1500) * 0.25).astype(np.float32)
    ex = np.sort(rng.choice(1500, 300, replace=False))
    got = O.importance_topk(g, 200, exclude=ex)
    assert np.array_equal(got, brute_topk(g, 200, ex))
    assert np.intersect1d(got, ex).size == 0


def test_rigl_brute_force_and_invariants():
    rng = np.random.default_rng(12)
    N, k = 2000, 100
    r = (3 * k) // 10
    g = (rng.integers(0, 5, N) * 0.1).astype(np.float32)
    w = O.bf16_rne(rng.integers(-3, 4, N) * 0.01)
    S_old = np.sort(rng.choice(N, k, replace=False)).astype(np.uint32)
    m = rng.standard_normal(k); v = rng.random(k)
    out = O.rigl_reselect(g, w, S_old, m, v, k, r)
    # drop: r lowest |w| among S_old, ties lowest index
    order = sorted(S_old.tolist(), key=lambda f: (abs(w[f]), f))
    D = sorted(order[:r])
    G = brute_topk(g, r, S_old).tolist()
    assert out["dropped"].tolist() == D and out["grown"].tolist() == G
    want = sorted(set(S_old.tolist()) - set(D) | set(G))
    assert out["S_new"].tolist() == want and len(want) == k
    assert set(D) <= set(S_old.tolist()) and not set(G) & set(S_old.tolist())
    pos_old = {f: i for i, f in enumerate(S_old.tolist())}
    for i, f in enumerate(out["S_new"].tolist()):
        if f in pos_old:
            assert out["m"][i] == m[pos_old[f]] and out["v"][i] == v[pos_old[f]]
        else:
            assert out["m"][i] == 0 and out["v"][i] == 0
    kept = sorted(set(S_old.tolist()) - set(D))
    assert max(abs(w[f]) for f in D) <= min(abs(w[f]) for f in kept)
    assert out["topk_new_vs_old"] == len(set(brute_topk(g, k).tolist()) - set(S_old.tolist()))


# --------------------------------------------------------------------------
# sequencing: NaN rule, frozen entries bit-identical
# --------------------------------------------------------------------------
def _step_inputs():
    d = synth.moe_layer(32, 16, 4, 2, 8, bf16=True, seeds=(20, 21, 22, 23, 24))
    shape = O.Shape(32, 16, 4, 2, 8)
    idx = synth.random_mask(shape.N, 40, 25)
    return d, shape, idx


def test_step_updates_only_listed_entries():
    import hashlib
    d, shape, idx = _step_inputs()
    z = np.zeros(idx.size)
    out = O.train_step(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], 2, idx, z, z,
                       np.zeros_like(d["Wr"]), np.zeros_like(d["Wr"]), 0, 1e-3, 0.9, 0.999,
                       1e-8, CB16)
    before = synth.flat_weights(d["W_gu"], d["W_d"]).astype(np.float64)
    frozen = np.ones(shape.N, bool); frozen[idx] = False
    h = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    assert h(out["W_flat"][frozen]) == h(before[frozen])
    assert out["t"] == 1 and not out["skipped"]
    assert np.count_nonzero(out["W_flat"][idx] != before[idx]) > 0.9 * idx.size


def test_nan_step_is_skipped_bit_identically():
    d, shape, idx = _step_inputs()
    d["tgt"] = d["tgt"].copy(); d["tgt"][3, 5] = np.nan
    m = np.arange(idx.size) * 1e-3; v = np.arange(idx.size) * 1e-6
    mr = np.ones_like(d["Wr"]); vr = np.ones_like(d["Wr"])
    out = O.train_step(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], 2, idx, m, v, mr, vr, 7,
                       1e-3, 0.9, 0.999, 1e-8, CB16)
    assert out["skipped"] and out["t"] == 7
    assert np.array_equal(out["W_flat"], synth.flat_weights(d["W_gu"], d["W_d"]))
    assert np.array_equal(out["m"], m) and np.array_equal(out["v"], v)
    assert np.array_equal(out["Wr"], d["Wr"]) and np.array_equal(out["mr"], mr)


# --------------------------------------------------------------------------
# numbers printed on the pages
# --------------------------------------------------------------------------
def test_page_parameter_counts():
    with open(os.path.join(GOLDEN, "page_counts.json")) as f:
        gd = json.load(f)
    per_layer = O.n_expert_weights(gd["H"], gd["E"], gd["I"])
    n_train_layers = gd["n_layers"] - gd["train_from"]
    experts = per_layer * n_train_layers
    k = O.select_count(experts, gd["frac_num"], gd["frac_den"])
    router = n_train_layers * gd["E"] * gd["H"]
    assert abs(experts / gd["expert_weights_in_trainable_layers"] - 1) < gd["expert_weights_rel_tol"]
    assert abs(router / gd["router_params"] - 1) < gd["router_params_rel_tol"]
    assert abs((k + router) / gd["trainable_total"] - 1) < gd["trainable_total_rel_tol"]


def test_select_count_floor():
    assert O.select_count(49152, 5, 100) == 2457
    assert O.select_count(603979776, 5, 1000) == 3019898
    assert O.select_count(1409286144, 5, 1000) == 7046430
    assert O.select_count(3019898 , 3, 10) == 905969

"""GPU parity on the method's degenerate cases: an empty active list, a single
token, a selection of nothing or of everything, and a RigL step that moves
no entry.  Same bars as the other parity tests: integer results bit-exact,
floating point within 1e-4 (fp32) or 2e-2 (bf16) of max|ref|."""
import numpy as np
import pytest
import torch

import usaf_synth as synth
from oracle import usaf_oracle as O
from test_gpu_parity import TOL_BF16, TOL_F32, npf, npu32, oracle_layer, rel, run_layer, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def capi():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_fine_tuning_amd import capi as c
    return c


def check_layer(lay, ref, act, dense=None):
    tol = TOL_BF16 if act else TOL_F32
    fw, bw = ref["fw"], ref["bw"]
    assert np.array_equal(lay.st["topk_ids"].cpu().numpy(), fw["topk_ids"])
    assert np.array_equal(lay.st["offsets"].cpu().numpy(), fw["offsets"])
    assert rel(npf(lay.Y), fw["Y"]) <= tol
    assert rel(npf(lay.dWr), bw["dWr"]) <= tol
    assert rel(npf(lay.dX), bw["dX"]) <= tol
    if dense is not None:
        assert rel(npf(dense), ref["gd"]) <= tol


@pytest.mark.parametrize("act", [1, 0])
def test_empty_active_list(capi, act):
    """No selected entry: the step still routes, runs the experts and trains
    the router; no expert weight moves."""
    say(f"empty active list act={act}")
    dims = (200, 128, 8, 2, 96)
    d = synth.moe_layer(*dims, bf16=bool(act), seeds=(120, 121, 122, 123, 124))
    idx = np.zeros(0, np.uint32)
    lay, _ = run_layer(capi, d, dims, act, idx)
    ref = oracle_layer(d, dims, act, idx)
    assert ref["g"].size == 0 and lay.dW.numel() == 0
    check_layer(lay, ref, act)
    assert int(lay.nonfinite.item()) == 0
    W0, Wr0 = lay.W.clone(), lay.Wr.clone()
    lay.train_step(lr=1e-3)
    torch.cuda.synchronize()
    assert torch.equal(lay.W, W0)
    assert not torch.equal(lay.Wr, Wr0)
    assert lay.t == 1


@pytest.mark.parametrize("act", [1, 0])
def test_single_token(capi, act):
    """T = 1: K experts hold one slot each, every other expert is empty."""
    say(f"single token act={act}")
    dims = (1, 64, 8, 2, 32)
    T, H, E, K, I = dims
    d = synth.moe_layer(*dims, bf16=bool(act), seeds=(130, 131, 132, 133, 134))
    N = 3 * E * H * I
    idx = synth.random_mask(N, N // 50, 135)
    lay, dense = run_layer(capi, d, dims, act, idx, dense=True)
    ref = oracle_layer(d, dims, act, idx)
    check_layer(lay, ref, act, dense)
    assert rel(npf(lay.dW), ref["g"]) <= (TOL_BF16 if act else TOL_F32)


def run_topk(capi, g, k, ex=None):
    n = g.size
    gt = torch.from_numpy(g).to(DEV)
    ext = None if ex is None else torch.from_numpy(ex.view(np.int32)).to(DEV)
    out = torch.full((max(k, 1),), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(capi.workspace_size(capi.WS_TOPK, None, n), dtype=torch.uint8, device=DEV)
    capi.importance_topk(gt, n, k, ext, 0 if ex is None else ex.size, out, None, ws)
    torch.cuda.synchronize()
    return npu32(out)


def test_topk_nothing_and_everything(capi):
    say("topk k = 0, k = n, k = n - n_exclude")
    rng = np.random.default_rng(140)
    n = 5000
    g = (rng.integers(-3, 4, n) * 0.5).astype(np.float32)
    # k = 0 selects nothing and leaves the output alone
    assert npu32(torch.full((1,), -7, dtype=torch.int32)).tolist() == run_topk(capi, g, 0).tolist()
    # k = n selects every index
    assert np.array_equal(run_topk(capi, g, n), np.arange(n, dtype=np.uint32))
    # k = n - n_exclude selects exactly the complement of the exclusion
    ex = np.sort(rng.choice(n, 777, replace=False)).astype(np.uint32)
    want = np.setdiff1d(np.arange(n, dtype=np.uint32), ex)
    got = run_topk(capi, g, n - ex.size, ex)
    assert np.array_equal(got, want)
    assert np.array_equal(got, O.importance_topk(g, n - ex.size, exclude=ex))


@pytest.mark.parametrize("act", [1, 0])
def test_rigl_moves_nothing_at_r_zero(capi, act):
    say(f"rigl r = 0 act={act}")
    T, H, E, K, I = 16, 64, 4, 2, 32
    N = 3 * E * H * I
    k = 1000
    rng = np.random.default_rng(150 + act)
    g = rng.standard_normal(N).astype(np.float32)
    w = (rng.integers(-6, 7, N) * 0.0078125).astype(np.float32)
    S_old = synth.random_mask(N, k, 151)
    m = rng.standard_normal(k).astype(np.float32)
    v = rng.random(k).astype(np.float32)
    Wt = torch.from_numpy(w).to(DEV)
    if act:
        Wt = Wt.to(torch.bfloat16)
    new_idx = torch.empty(k, dtype=torch.int32, device=DEV)
    new_m = torch.empty(k, dtype=torch.float32, device=DEV)
    new_v = torch.empty(k, dtype=torch.float32, device=DEV)
    stats = torch.zeros(3, dtype=torch.int64, device=DEV)
    ws = torch.empty(capi.workspace_size(capi.WS_RIGL, None, N, k), dtype=torch.uint8, device=DEV)
    capi.rigl_reselect(capi.Shape(T, H, E, K, I, act), torch.from_numpy(g).to(DEV), Wt,
                       torch.from_numpy(S_old.view(np.int32)).to(DEV), torch.from_numpy(m).to(DEV),
                       torch.from_numpy(v).to(DEV), k, 0, new_idx, new_m, new_v, stats, ws)
    torch.cuda.synchronize()
    ref = O.rigl_reselect(g, w, S_old, m, v, k, 0)
    assert np.array_equal(npu32(new_idx), S_old)
    assert np.array_equal(ref["S_new"], S_old)
    assert np.array_equal(new_m.cpu().numpy(), m)
    assert np.array_equal(new_v.cpu().numpy(), v)
    s = stats.cpu().numpy()
    assert s[0] == 0 and s[1] == 0 and s[2] == ref["topk_new_vs_old"]

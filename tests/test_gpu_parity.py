"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer work (routing ids, grouping, selections, RigL sets) must match
bit-exactly given identical inputs; floating point within
max|gpu - ref| / max|ref| <= 1e-4 for fp32 layers and 2e-2 for bf16 layers.
"""
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


def bf16_bits(x64):
    return (np.asarray(x64, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# a1 dequant
# --------------------------------------------------------------------------
@pytest.mark.parametrize("rows,cols", [(96, 384), (1, 64), (513, 768)])
def test_dequant_bit_exact(capi, rows, cols):
    say(f"dequant rows={rows} cols={cols}")
    rng = np.random.default_rng(rows + cols)
    q = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    mags = np.concatenate([np.array([0.0, 5.96e-8, 6.1e-5, 65504.0]),
                           10.0 ** rng.uniform(-7, 4, 1000)])
    sc = (rng.choice(mags, size=(rows, cols // 64)) * rng.choice([-1, 1], size=(rows, cols // 64)))
    sc = sc.astype(np.float16)
    qt = torch.from_numpy(q).to(DEV)
    st = torch.from_numpy(sc.view(np.int16)).to(DEV)
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device=DEV)
    capi.dequant_resident(qt, st, rows, cols, 64, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = O.dequant_int4(q, sc.view(np.uint16))
    assert np.array_equal(got, bf16_bits(ref))


@pytest.mark.parametrize("rows,cols,group", [(96, 384, 128), (1, 128, 128), (513, 768, 64),
                                            (64, 2048, 128)])
def test_dequant_affine_bit_exact(capi, rows, cols, group):
    """The HQQ-style affine storage: unsigned codes, fp16 scale and zero per group."""
    say(f"dequant affine rows={rows} cols={cols} group={group}")
    rng = np.random.default_rng(rows + cols + group)
    q = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    ng = (rows, cols // group)
    mags = np.concatenate([np.array([0.0, 5.96e-8, 6.1e-5, 65504.0]), 10.0 ** rng.uniform(-7, 4, 1000)])
    sc = (rng.choice(mags, size=ng) * rng.choice([-1, 1], size=ng)).astype(np.float16)
    zr = np.concatenate([np.array([0.0, -(2.0 ** -24), 7.5, 65504.0]), rng.uniform(-4, 20, 1000)])
    zr = rng.choice(zr, size=ng).astype(np.float16)
    out = torch.empty(rows, cols, dtype=torch.bfloat16, device=DEV)
    capi.dequant_affine(torch.from_numpy(q).to(DEV), torch.from_numpy(sc.view(np.int16)).to(DEV),
                        torch.from_numpy(zr.view(np.int16)).to(DEV), rows, cols, group, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = O.dequant_affine(q, sc.view(np.uint16), zr.view(np.uint16), group)
    assert np.array_equal(got, bf16_bits(ref))


# --------------------------------------------------------------------------
# a3-a4 routing from given logits
# --------------------------------------------------------------------------
def route_state(T, E, K):
    S = T * K
    z = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device=DEV)
    return dict(topk_ids=z(T, K), topk_w=z(T, K, dt=torch.float32), offsets=z(E + 1),
                perm=z(S), slot_pos=z(S))


@pytest.mark.parametrize("T,E,K,ties", [(300, 128, 8, False), (300, 128, 8, True),
                                        (77, 8, 2, True), (50, 5, 5, False), (5, 1024, 64, True),
                                        (4096, 128, 8, True), (2048, 1024, 8, False),
                                        (100, 1, 1, False), (1500, 200, 3, True)])
def test_route_exact_given_logits(capi, T, E, K, ties):
    say(f"route T={T} E={E} K={K} ties={ties}")
    rng = np.random.default_rng(T * E + K)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if ties:
        logits = (np.round(logits * 2) / 2).astype(np.float32)
        logits[0, :] = 0.0
        logits[1, ::2] = -0.0
    shape = capi.Shape(T, 64, E, K, 32, capi.F32)
    d = route_state(T, E, K)
    capi.route(shape, torch.from_numpy(logits).to(DEV), capi.make_state(d))
    torch.cuda.synchronize()
    R = O.Rounding(O.F32, O.CONTRACT)
    ids, w = O.route_topk(logits, K, R)
    counts, offsets, perm = O.group_by_expert(ids, E)
    assert np.array_equal(d["topk_ids"].cpu().numpy(), ids)
    assert np.array_equal(d["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(d["perm"].cpu().numpy(), perm)
    inv = np.empty_like(perm); inv[perm] = np.arange(perm.size)
    assert np.array_equal(d["slot_pos"].cpu().numpy(), inv)
    assert rel(npf(d["topk_w"]), w) <= 1e-6


# --------------------------------------------------------------------------
# a2-a13: forward + backward of one layer
# --------------------------------------------------------------------------
def run_layer(capi, d, dims, act, idx, dense=False):
    from sparse_fine_tuning_amd.layer import SparseMoELayer
    T, H, E, K, I = dims
    lay = SparseMoELayer(T, H, E, K, I, act=act, device=DEV)
    lay.load(d["X"], d["Wr"], d["W_gu"], d["W_d"], d["tgt"])
    lay.set_active(idx)
    lay.forward()
    lay.loss_grad()
    lay.backward()
    dense_out = None
    if dense:
        dense_out = torch.empty(lay.shape.N, dtype=torch.float32, device=DEV)
        dx_keep = lay.dX.clone()
        lay.backward(dense_out=dense_out, want_dx=False)
        lay.dX.copy_(dx_keep)
    torch.cuda.synchronize()
    return lay, dense_out


def oracle_layer(d, dims, act, idx):
    T, H, E, K, I = dims
    R = O.Rounding(O.BF16 if act else O.F32, O.CONTRACT)
    shape = O.Shape(*dims)
    fw = O.moe_forward(d["X"], d["Wr"], d["W_gu"], d["W_d"], K, R)
    loss, dY = O.mse_loss_grad(fw["Y"], d["tgt"], R)
    bw = O.moe_backward(fw, d["X"], d["Wr"], d["W_gu"], d["W_d"], dY, R)
    g = O.weight_grads_at(fw, bw, d["X"], dY, idx, shape, R)
    gd = O.weight_grads_dense(fw, bw, d["X"], dY, shape, R)
    return dict(fw=fw, bw=bw, loss=loss, dY=dY, g=g, gd=gd)


CASES = [
    # name, dims, act, seeds, weight scale
    ("tiny_fp32", (128, 64, 8, 2, 32), 0, (0, 1, 2, 3, 4)),
    ("ragged_fp32", (200, 128, 6, 3, 96), 0, (30, 31, 32, 33, 34)),
    ("empty_experts_fp32", (8, 64, 16, 1, 32), 0, (40, 41, 42, 43, 44)),
    ("ragged_bf16", (200, 128, 8, 2, 96), 1, (50, 51, 52, 53, 54)),
    # the MFMA path with most experts empty: one token (two slots), and eight
    # tokens over sixteen experts
    ("single_token_bf16", (1, 128, 8, 2, 64), 1, (45, 46, 47, 48, 49)),
    ("empty_experts_bf16", (8, 128, 16, 1, 64), 1, (40, 41, 42, 43, 44)),
    # every token routed to every expert (K = E): equal groups of T slots
    ("all_experts_bf16", (96, 128, 4, 4, 64), 1, (35, 36, 37, 38, 39)),
    ("wide_bf16", (333, 256, 16, 4, 160), 1, (60, 61, 62, 63, 64)),
    # column-tiled masked gradient: gate_up has H > 2048 columns, down has I > 2048
    ("coltiled_gate_up_bf16", (64, 4096, 4, 2, 64), 1, (70, 71, 72, 73, 74)),
    ("coltiled_down_bf16", (48, 128, 3, 2, 2560), 1, (80, 81, 82, 83, 84)),
    # >= 512 rows per expert on average: the 256-row GEMM tiles, ragged
    ("big_groups_bf16", (1100, 256, 4, 2, 96), 1, (85, 86, 87, 88, 89)),
    # 160-row GEMM tiles split evenly: groups of ~300 rows take 160 + the
    # rest, the two wave-rows sharing 5 blocks 3 + 2
    ("row_tiles_bf16", (600, 128, 4, 2, 96), 1, (95, 96, 97, 98, 99)),
    # groups of ~350 rows: three tiles of 128, 128 and the rest
    ("row_tiles_350_bf16", (700, 128, 4, 2, 64), 1, (115, 116, 117, 118, 119)),
    # groups of 161..192 rows: two tiles of 96 + the rest
    ("row_tiles_180_bf16", (360, 128, 4, 2, 64), 1, (105, 106, 107, 108, 109)),
    # the down and dX launches end on a short round of tiles, whose
    # contraction is split over the idle blocks (256 CUs): 256-row tiles,
    # 64 tail tiles in 2 parts
    ("tail_split_big_bf16", (2200, 4096, 4, 2, 256), 1, (120, 121, 122, 123, 124)),
    # 160-row tiles, 8 tail tiles in 4 parts (one stage each for down)
    ("tail_split_bf16", (2000, 2048, 24, 4, 256), 1, (130, 131, 132, 133, 134)),
    # 3 parts, the last one ragged (I = 160: 64 + 64 + 32)
    ("tail_split_ragged_k_bf16", (1200, 4096, 18, 2, 160), 1, (130, 131, 132, 133, 134)),
    # gate_up split in 2 parts and dA in 4 (160-row tiles)
    ("tail_split_gate_up_da_bf16", (1024, 1024, 17, 4, 2048), 1, (150, 151, 152, 153, 154)),
    # experts of 8344, 8053 and 8203 slots: the dense dW contracts over 250+
    # stages of 32 slots, the grouped GEMMs run 32-33 row tiles per expert
    ("long_groups_bf16", (12300, 128, 3, 2, 64), 1, (160, 161, 162, 163, 164)),
]


def row_tile(BM, cnt):
    """Rows per tile of a group of cnt rows (the GEMMs' grouped tiling)."""
    if (BM // 32) % 2 == 0:
        return BM
    n = (cnt + BM - 1) // BM
    return ((cnt + n - 1) // n + 31) // 32 * 32 if n > 0 else BM


def tail_split_parts(offsets, dims, gemm):
    """Parts per tail tile of a bf16 grouped GEMM launch ("gate_up", "down",
    "da" or "dx") on this device: 1 when the launch runs unsplit.  The
    launch has one block per CU (these tile shapes fill a CU's LDS); its last
    round of tiles, when at most half full, is split into S <= 4 parts,
    bounded by the partial buffer (the [T K, H] fp32-sized region for
    gate_up and dA, its spare half for down and dX, less 256 bytes) and the
    contraction's 64-wide stages."""
    T, H, E, K, I = dims
    big = T * K >= 512 * E and gemm != "da"
    BM, IM = (256, 4) if big else (160, 3)
    NT, contraction, room = {"gate_up": ((I + 127) // 128, H, 4), "down": ((H + 255) // 256, I, 2),
                             "da": ((I + 255) // 256, H, 4), "dx": ((H + 255) // 256, 2 * I, 2)}[gemm]
    cnt = np.diff(offsets)
    tiles = int(sum(((c + row_tile(BM, c) - 1) // row_tile(BM, c)) * NT for c in cnt if c > 0))
    G = (torch.cuda.get_device_properties(0).multi_processor_count + 7) // 8 * 8
    cap = (T * K * H * room - 256) // (512 * IM * 2 * 64)
    R, rem = divmod(tiles, G)
    if cap < 2 or R < 1 or rem == 0 or 2 * rem > G:
        return 1
    S = min(4, G // rem, cap // rem, (contraction + 63) // 64)
    return S if S >= 2 else 1


@pytest.mark.parametrize("name,dims,act,seeds", CASES, ids=[c[0] for c in CASES])
def test_layer_forward_backward(capi, name, dims, act, seeds):
    say(f"layer {name} dims={dims} act={act}")
    T, H, E, K, I = dims
    d = synth.moe_layer(T, H, E, K, I, bf16=bool(act), seeds=seeds)
    N = 3 * E * H * I
    idx = synth.random_mask(N, max(1, N // 50), seeds[0] + 100)
    lay, dense = run_layer(capi, d, dims, act, idx, dense=True)
    ref = oracle_layer(d, dims, act, idx)
    tol = TOL_BF16 if act else TOL_F32
    fw, bw = ref["fw"], ref["bw"]
    st = lay.st
    # routing and grouping: exact (GPU logits equal up to rounding; no near-ties at these seeds)
    ids = st["topk_ids"].cpu().numpy()
    assert np.array_equal(ids, fw["topk_ids"]), "routing differs"
    assert np.array_equal(st["offsets"].cpu().numpy(), fw["offsets"])
    if name.startswith("tail_split") and torch.cuda.get_device_properties(0).multi_processor_count == 256:
        parts = {g: tail_split_parts(fw["offsets"], dims, g) for g in ("gate_up", "down", "da", "dx")}
        say(f"  tail split parts: {parts}")
        want = ("gate_up", "da") if "gate_up_da" in name else ("down", "dx")
        assert min(parts[g] for g in want) >= 2, "the case no longer exercises the tail split"
    perm = st["perm"].cpu().numpy()
    assert np.array_equal(perm, fw["perm"])
    assert rel(npf(st["logits"]), fw["logits"]) <= tol
    assert rel(npf(st["topk_w"]), fw["topk_w"]) <= tol
    # saved activations are expert-major: row p holds slot perm[p]
    assert rel(npf(st["gu"]), fw["gu"][perm]) <= tol
    assert rel(npf(st["a"]), fw["a"][perm]) <= tol
    assert rel(npf(lay.Y), fw["Y"]) <= tol
    assert abs(float(lay.loss.item()) - ref["loss"]) <= tol * abs(ref["loss"])
    assert rel(npf(lay.dY), ref["dY"]) <= tol
    assert rel(npf(st["dgu"]), bw["dgu"][perm]) <= tol
    assert rel(npf(st["dw"]), bw["dw"]) <= tol
    assert rel(npf(lay.dWr), bw["dWr"]) <= tol
    assert rel(npf(lay.dX), bw["dX"]) <= tol
    assert rel(npf(lay.dW), ref["g"]) <= tol
    assert rel(npf(dense), ref["gd"]) <= tol
    assert int(lay.nonfinite.item()) == 0


def test_masked_at_full_density_equals_dense(capi):
    say("masked dW at 100% density")
    dims = (64, 2048, 2, 1, 64)
    d = synth.moe_layer(*dims, bf16=True, seeds=(90, 91, 92, 93, 94))
    N = 3 * 2 * 2048 * 64
    idx = np.arange(N, dtype=np.uint32)
    lay, dense = run_layer(capi, d, dims, 1, idx, dense=True)
    g = npf(lay.dW)
    ref = oracle_layer(d, dims, 1, idx[:1])["gd"]
    assert rel(g, ref) <= TOL_BF16
    assert rel(g, npf(dense)) <= TOL_BF16


def skewed_mask(kind, dims, gd):
    """Clustered active lists: an importance selection (top-2% of the dense
    gradient: a few rows carry most entries), whole rows at unaligned
    positions over sparse entries, or every entry in one expert."""
    T, H, E, K, I = dims
    N = 3 * E * H * I
    ngu = E * 2 * I * H
    rng = np.random.default_rng(11)
    if kind == "importance":
        return O.importance_topk(gd, N // 50)
    if kind == "rows":
        rows = [(1, 3), (1, 4), (1, 5), (1, 1001), (2, 2 * I - 1), (0, 517)]  # (expert, gate_up row)
        full = [np.arange(H, dtype=np.int64) + (e * 2 * I + r) * H for e, r in rows]
        down_rows = [(3, 9), (3, 10)]
        full += [ngu + np.arange(I, dtype=np.int64) + (e * H + r) * I for e, r in down_rows]
        sparse = rng.choice(N, N // 500, replace=False)
        return np.unique(np.concatenate(full + [sparse])).astype(np.uint32)
    if kind == "one_expert":
        e = 2
        gu = np.arange(e * 2 * I * H, (e + 1) * 2 * I * H, dtype=np.int64)
        dn = ngu + np.arange(e * H * I, (e + 1) * H * I, dtype=np.int64)
        pool = np.concatenate([gu, dn])
        return np.sort(rng.choice(pool, pool.size * 3 // 10, replace=False)).astype(np.uint32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["importance", "rows", "one_expert"])
def test_masked_dw_clustered_lists(capi, kind):
    """The masked gradient on lists far from uniform: the tiles follow the
    entry counts, so heavy rows and experts are split and empty ones skipped."""
    dims = (256, 2048, 4, 2, 256)
    say(f"masked dW clustered list {kind} dims={dims}")
    d = synth.moe_layer(*dims, bf16=True, seeds=(120, 121, 122, 123, 124))
    gd = oracle_layer(d, dims, 1, np.zeros(1, np.uint32))["gd"]
    idx = skewed_mask(kind, dims, gd)
    lay, _ = run_layer(capi, d, dims, 1, idx, dense=False)
    got = npf(lay.dW)
    want = gd[idx.astype(np.int64)]
    assert rel(got, want) <= TOL_BF16
    assert int(lay.nonfinite.item()) == 0


def test_kept_plan_equals_plan_per_call(capi):
    """usaf_masked_backward with the plan usaf_masked_plan kept for the list
    gives the same bits as with the plan rebuilt inside the call, also after
    the list (and so the plan) changes."""
    dims = (256, 2048, 4, 2, 256)
    say(f"kept masked plan dims={dims}")
    d = synth.moe_layer(*dims, bf16=True, seeds=(120, 121, 122, 123, 124))
    N = 3 * 4 * 2048 * 256
    for mask_seed in (3, 4):
        idx = synth.random_mask(N, N // 100, mask_seed)
        lay, _ = run_layer(capi, d, dims, 1, idx, dense=False)  # the layer keeps a plan
        kept = lay.dW.clone()
        capi.masked_backward(lay.shape, lay.X, lay.Wr, lay.W, lay.state, lay.dY, lay.idx,
                             lay.idx.numel(), lay.dW, lay.dWr, None, None, lay.ws_bwd)
        torch.cuda.synchronize()
        assert torch.equal(kept, lay.dW)


def test_repeat_runs_are_bit_identical(capi):
    say("determinism ragged_bf16")
    dims = (200, 128, 8, 2, 96)
    d = synth.moe_layer(*dims, bf16=True, seeds=(50, 51, 52, 53, 54))
    idx = synth.random_mask(3 * 8 * 128 * 96, 3000, 7)
    a, da = run_layer(capi, d, dims, 1, idx, dense=True)
    b, db = run_layer(capi, d, dims, 1, idx, dense=True)
    for x, y in ((a.Y, b.Y), (a.dX, b.dX), (a.dW, b.dW), (a.dWr, b.dWr), (da, db),
                 (a.st["dw"], b.st["dw"])):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


# --------------------------------------------------------------------------
# a14 top-k, a15 RigL
# --------------------------------------------------------------------------
TOPK_CASES = [(10000, 500, "normal"), (50000, 12345, "ties"), (4096 * 3 + 17, 4096 * 3 + 17, "normal"),
              (9999, 1, "ties"), (200000, 1000, "exclude"), (100000, 3000, "ties_exclude"),
              (1, 1, "normal"), (2, 1, "allsame"), (3, 2, "ties"),
              (4096, 4000, "allsame"), (123457, 61728, "exclude"),
              # from 2^20 keys on, a whole gradient takes the sampled single pass
              (3000001, 15000, "normal"), (2500000, 200000, "ties"), (1 << 20, 1 << 20, "normal"),
              (1500003, 1000, "allsame"), (1 << 21, 3, "normal"),
              (2097152 + 4093, 100000, "sample_misleads"), (2 ** 21, 5000, "sample_floods"),
              (2000000, 30000, "exclude")]


@pytest.mark.parametrize("n,k,mode", TOPK_CASES)
def test_topk_exact(capi, n, k, mode):
    say(f"topk n={n} k={k} mode={mode}")
    rng = np.random.default_rng(n + k)
    g = rng.standard_normal(n).astype(np.float32)
    if "ties" in mode:
        g = (rng.integers(-3, 4, n) * 0.25).astype(np.float32)
    if mode == "allsame":
        g = np.full(n, -0.5, np.float32)
    sampled = np.arange(n) % 256 < 4  # the keys the sampled pass histograms
    if mode == "sample_misleads":
        # the sample sees only large keys, so its threshold lets through
        # fewer than k keys: the pass must run again with every key
        g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        g[sampled] = np.float32(10.0) + rng.random(np.count_nonzero(sampled)).astype(np.float32)
    if mode == "sample_floods":
        # the sample sees only small keys: nearly every key is a candidate
        g = (rng.standard_normal(n) + 5.0).astype(np.float32)
        g[sampled] = (rng.standard_normal(np.count_nonzero(sampled)) * 1e-3).astype(np.float32)
    ex = None
    if "exclude" in mode:
        ex = np.sort(rng.choice(n, n // 10, replace=False)).astype(np.uint32)
    gt = torch.from_numpy(g).to(DEV)
    ext = None if ex is None else torch.from_numpy(ex.view(np.int32)).to(DEV)
    out = torch.empty(k, dtype=torch.int32, device=DEV)
    val = torch.empty(k, dtype=torch.float32, device=DEV)
    ws = torch.empty(capi.workspace_size(capi.WS_TOPK, None, n), dtype=torch.uint8, device=DEV)
    capi.importance_topk(gt, n, k, ext, 0 if ex is None else ex.size, out, val, ws)
    torch.cuda.synchronize()
    ref = O.importance_topk(g, k, exclude=ex)
    got = npu32(out)
    assert np.array_equal(got, ref)
    assert np.array_equal(val.cpu().numpy(), g[ref])


@pytest.mark.parametrize("act,old_is_top,dims", [
    (1, False, (16, 64, 4, 2, 32)), (0, False, (16, 64, 4, 2, 32)), (1, True, (16, 64, 4, 2, 32)),
    # N = 12.6M: the sampled fresh top-k and the merges over 31 blocks of the old list
    (1, False, (16, 1024, 8, 2, 512)), (1, True, (16, 1024, 8, 2, 512))])
def test_rigl_exact(capi, act, old_is_top, dims):
    """old_is_top: the old set holds the largest |g|, so fewer than r entries of
    a fresh top-k are new and the grow set must come from the full selection
    that excludes the old set."""
    say(f"rigl act={act} old_is_top={old_is_top} dims={dims}")
    T, H, E, K, I = dims
    N = 3 * E * H * I
    k = 1000 if N < 100000 else O.select_count(N, 5, 1000)
    r = (3 * k) // 10
    rng = np.random.default_rng(17 + act)
    g = (rng.integers(-4, 5, N) * 0.125).astype(np.float32)
    w = (rng.integers(-6, 7, N) * 0.0078125).astype(np.float32)  # exact in bf16, many ties
    S_old = synth.random_mask(N, k, 3)
    if old_is_top:
        g[S_old] = np.float32(4.0) * np.sign(g[S_old] + 0.01)
    m = rng.standard_normal(k).astype(np.float32)
    v = rng.random(k).astype(np.float32)
    shape = capi.Shape(T, H, E, K, I, act)
    Wt = torch.from_numpy(w).to(DEV)
    if act:
        Wt = Wt.to(torch.bfloat16)
    new_idx = torch.empty(k, dtype=torch.int32, device=DEV)
    new_m = torch.empty(k, dtype=torch.float32, device=DEV)
    new_v = torch.empty(k, dtype=torch.float32, device=DEV)
    stats = torch.zeros(3, dtype=torch.int64, device=DEV)
    ws = torch.empty(capi.workspace_size(capi.WS_RIGL, None, N, k), dtype=torch.uint8, device=DEV)
    old_t = torch.from_numpy(S_old.view(np.int32)).to(DEV)
    g_t = torch.from_numpy(g).to(DEV)
    ref = O.rigl_reselect(g, w, S_old, m, v, k, r)
    # drop keys gathered from the flat weights, then read from a compact copy
    # of them at the old list (SparseAdam's list)
    old_w = torch.empty(k, dtype=Wt.dtype, device=DEV)
    capi.gather(act, Wt, old_t, k, old_w)
    new_w = torch.empty_like(old_w)
    for ow in (None, old_w):
        stats.zero_()
        capi.rigl_reselect(shape, g_t, Wt, old_t, torch.from_numpy(m).to(DEV),
                           torch.from_numpy(v).to(DEV), k, r, new_idx, new_m, new_v, stats, ws,
                           old_w=ow, new_w=None if ow is None else new_w)
        torch.cuda.synchronize()
        assert np.array_equal(npu32(new_idx), ref["S_new"])
        if ow is not None:  # the new compact list is W at the new list
            want = torch.empty_like(old_w)
            capi.gather(act, Wt, new_idx, k, want)
            assert torch.equal(new_w, want)
        assert np.array_equal(new_m.cpu().numpy(), ref["m"].astype(np.float32))
        assert np.array_equal(new_v.cpu().numpy(), ref["v"].astype(np.float32))
        s = stats.cpu().numpy()
        assert s[0] == r and s[1] == r and s[2] == ref["topk_new_vs_old"]
    assert (ref["topk_new_vs_old"] < r) == old_is_top


# --------------------------------------------------------------------------
# a12 Adam and the NaN skip
# --------------------------------------------------------------------------
@pytest.mark.parametrize("act,use_list", [(1, False), (0, False), (1, True), (0, True)])
def test_sparse_adam(capi, act, use_list):
    say(f"adam act={act} list={use_list}")
    rng = np.random.default_rng(5 + act)
    N, k = 50000, (4001 if use_list else 4000)  # 4001: the list kernel's 4-wide tail
    w = synth.normal(N, 0.02, 9)
    if act:
        w = synth.to_bf16_values(w)
    idx = synth.random_mask(N, k, 10)
    R = O.Rounding(O.BF16 if act else O.F32, O.CONTRACT)
    m = np.zeros(k); v = np.zeros(k)
    Wt = torch.from_numpy(w).to(DEV)
    if act:
        Wt = Wt.to(torch.bfloat16)
    mt = torch.zeros(k, device=DEV); vt = torch.zeros(k, device=DEV)
    it = torch.from_numpy(idx.view(np.int32)).to(DEV)
    wl = None
    if use_list:
        wl = torch.empty(k, dtype=Wt.dtype, device=DEV)
        capi.gather(act, Wt, it, k, wl)
    wref = w.astype(np.float64)
    for step in range(1, 4):
        g = (rng.standard_normal(k) * 10.0 ** rng.integers(-8, -3, k)).astype(np.float32)
        capi.sparse_adam(act, Wt, it, k, torch.from_numpy(g).to(DEV), mt, vt, step, 1e-3, 0.9,
                         0.999, 1e-8, w_list=wl)
        wsel, m, v = O.adam_update(wref[idx], g, m, v, step, 1e-3, 0.9, 0.999, 1e-8,
                                   R.act_dtype, R)
        wref[idx] = wsel
    torch.cuda.synchronize()
    assert rel(mt.cpu().numpy(), m) <= 1e-5
    assert rel(vt.cpu().numpy(), v) <= 1e-5
    got = npf(Wt)
    frozen = np.ones(N, bool); frozen[idx] = False
    assert np.array_equal(got[frozen], w.astype(np.float64)[frozen])
    check_update(got[idx], wref[idx], w[idx], act)
    # the touched entries moved by ~lr per step
    assert np.median(np.abs(got[idx] - w[idx])) > 1e-3
    if use_list:  # the compact copy still equals W at idx
        assert torch.equal(wl, Wt[it.long()])


@pytest.mark.parametrize("act,n", [(1, 4001), (0, 4001), (1, 1), (1, 0), (0, 300000)])
def test_scatter_is_the_inverse_of_gather(capi, act, n):
    """usaf_scatter writes a compact list back at its indices (numpy's
    W[idx] = vals, bit for bit) and leaves every other weight alone; a
    gather followed by a scatter of the gathered list changes nothing."""
    say(f"scatter act={act} n={n}")
    N = 1 << 20
    w = synth.normal(N, 0.02, 30)
    if act:
        w = synth.to_bf16_values(w)
    idx = synth.random_mask(N, n, 31) if n else np.zeros(0, np.uint32)
    vals = synth.normal(max(n, 1), 1.0, 32)[:n]
    dt = torch.bfloat16 if act else torch.float32
    Wt = torch.from_numpy(w.astype(np.float32)).to(DEV).to(dt)
    W0 = Wt.clone()
    it = torch.from_numpy(idx.view(np.int32)).to(DEV)
    vt = torch.from_numpy(vals.astype(np.float32)).to(DEV).to(dt)
    capi.scatter(act, Wt, it, n, vt)
    back = torch.empty(n, dtype=dt, device=DEV)
    capi.gather(act, Wt, it, n, back)
    torch.cuda.synchronize()
    want = W0.clone()
    want[it.long() & 0xFFFFFFFF] = vt
    bits = (lambda x: x.view(torch.int16)) if act else (lambda x: x.view(torch.int32))
    assert torch.equal(bits(Wt), bits(want))
    assert torch.equal(bits(back), bits(vt))
    capi.scatter(act, Wt, it, n, back)  # the gathered list written back: no change
    torch.cuda.synchronize()
    assert torch.equal(bits(Wt), bits(want))


def check_update(w_gpu, w_ref, w_old, act):
    """The update itself, W_new - W_old, against the oracle's.  fp32: within
    the fp32 tolerance of max|dW|.  bf16: both sides round every step's
    result once to bf16 (fp32 vs fp64 arithmetic before it), so an entry may
    differ by at most one bf16 unit in the last place of its value, and only
    rarely; a wrong step size (half a step, a missing bias correction) moves
    nearly every entry."""
    d_gpu = np.asarray(w_gpu, np.float64) - w_old
    d_ref = np.asarray(w_ref, np.float64) - w_old
    if not act:
        assert rel(d_gpu, d_ref) <= TOL_F32
        return
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(w_ref), 1e-30))) - 7)
    diff = np.abs(d_gpu - d_ref)
    assert np.all(diff <= ulp * 1.0001), "an update differs by more than one bf16 ulp"
    assert np.count_nonzero(diff) <= 0.01 * diff.size, "updates differ in too many entries"


def test_new_weights_after_set_active_reach_adam(capi):
    """Weights loaded after the active list was set: SparseAdam must update
    the new weights, not the compact copy of the old ones."""
    say("weights replaced after set_active")
    from sparse_fine_tuning_amd.layer import SparseMoELayer
    dims = (200, 128, 8, 2, 96)
    T, H, E, K, I = dims
    d_old = synth.moe_layer(*dims, bf16=True, seeds=(40, 41, 42, 43, 44))
    d = synth.moe_layer(*dims, bf16=True, seeds=(50, 51, 52, 53, 54))
    N = 3 * E * H * I
    k = O.select_count(N, 5, 100)
    idx = synth.random_mask(N, k, 55)
    lay = SparseMoELayer(*dims, act=1, device=DEV)
    lay.load(d_old["X"], d_old["Wr"], d_old["W_gu"], d_old["W_d"], d_old["tgt"])
    lay.set_active(idx)
    lay.load(d["X"], d["Wr"], d["W_gu"], d["W_d"], d["tgt"])
    lay.train_step(lr=1e-3)
    torch.cuda.synchronize()
    assert lay.t == 1
    R = O.Rounding(O.BF16, O.CONTRACT)
    z = np.zeros(k)
    ref = O.train_step(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, idx, z, z,
                       np.zeros_like(d["Wr"]), np.zeros_like(d["Wr"]), 0, 1e-3, 0.9, 0.999,
                       1e-8, R)
    i64 = idx.astype(np.int64)
    w0 = np.concatenate([d["W_gu"].ravel(), d["W_d"].ravel()])
    got = npf(lay.W)
    # every entry moved from the new weights by about lr, in the oracle's direction
    sure = np.abs(ref["g"]) > TOL_BF16 * np.abs(ref["g"]).max()
    step = got[i64] - w0[i64]
    assert np.all(np.abs(step) <= 1e-3 * 1.01 + np.abs(w0[i64]) * 2.0 ** -7)
    assert np.all(np.sign(step[sure]) == np.sign(ref["W_flat"][i64][sure] - w0[i64][sure]))
    assert rel(got[i64][sure], ref["W_flat"][i64][sure]) <= TOL_BF16
    frozen = np.ones(N, bool); frozen[i64] = False
    assert np.array_equal(got[frozen], w0[frozen])
    assert torch.equal(lay.w_list, lay.W[lay.idx.long() & 0xFFFFFFFF])


def test_stale_plan_skips_the_step(capi):
    """A masked-gradient plan built for another list is recognised on the
    device: no gradient is written and the step is counted non-finite, so
    SparseAdam changes nothing."""
    say("stale plan")
    from sparse_fine_tuning_amd.layer import SparseMoELayer
    dims = (200, 128, 8, 2, 96)
    T, H, E, K, I = dims
    d = synth.moe_layer(*dims, bf16=True, seeds=(60, 61, 62, 63, 64))
    N = 3 * E * H * I
    lay = SparseMoELayer(*dims, act=1, device=DEV)
    lay.load(d["X"], d["Wr"], d["W_gu"], d["W_d"], d["tgt"])
    lay.set_active(synth.random_mask(N, 900, 65))
    old_plan = lay.plan.clone()
    lay.set_active(synth.random_mask(N, 1000, 66))
    lay.plan.copy_(old_plan)  # the kept plan now describes the first list
    W0 = lay.W.clone()
    lay.dW.fill_(7.0)
    lay.train_step(lr=1e-3)
    torch.cuda.synchronize()
    assert int(lay.nonfinite.item()) >= 1  # one count per gradient launch (gate_up, down)
    assert lay.skipped == 1 and lay.t == 0
    assert torch.all(lay.dW == 7.0)
    assert torch.equal(lay.W.view(torch.int16), W0.view(torch.int16))
    # the right plan again: a normal step
    lay.refresh_list()
    lay.train_step(lr=1e-3)
    torch.cuda.synchronize()
    assert int(lay.nonfinite.item()) == 0 and lay.t == 1


def test_nan_step_is_skipped(capi):
    say("nan skip")
    from sparse_fine_tuning_amd.layer import SparseMoELayer
    dims = (128, 64, 8, 2, 32)
    d = synth.moe_layer(*dims, bf16=True)
    d["tgt"] = d["tgt"].copy()
    d["tgt"][5, 7] = np.nan
    idx = synth.random_mask(3 * 8 * 64 * 32, 500, 1)
    lay = SparseMoELayer(*dims, act=1, device=DEV)
    lay.load(d["X"], d["Wr"], d["W_gu"], d["W_d"], d["tgt"])
    lay.set_active(idx)
    W0, Wr0 = lay.W.clone(), lay.Wr.clone()
    lay.m.fill_(0.5); lay.v.fill_(0.25)
    lay.train_step(lr=1e-3)
    torch.cuda.synchronize()
    assert lay.skipped == 1 and lay.t == 0
    assert torch.equal(lay.W.view(torch.int16), W0.view(torch.int16))
    assert torch.equal(lay.Wr, Wr0)
    assert torch.all(lay.m == 0.5) and torch.all(lay.v == 0.25)


# --------------------------------------------------------------------------
# the tiny fp32 workload end to end: importance pass, then 3 sparse steps
# --------------------------------------------------------------------------
def test_tiny_fp32_importance_then_three_steps(capi):
    say("tiny fp32 sequence")
    from sparse_fine_tuning_amd.layer import SparseMoELayer, topk
    dims = (128, 64, 8, 2, 32)
    T, H, E, K, I = dims
    d = synth.moe_layer(*dims, bf16=False)
    shape = O.Shape(*dims)
    k = O.select_count(shape.N, 5, 100)
    R = O.Rounding(O.F32, O.CONTRACT)
    # importance: the GPU computes its own gradients and selects
    lay = SparseMoELayer(*dims, act=0, device=DEV)
    lay.load(d["X"], d["Wr"], d["W_gu"], d["W_d"], d["tgt"])
    gdense = lay.dense_scan()
    sel_gpu = npu32(topk(gdense, k))
    sc = O.dense_scan(d["X"], d["tgt"], d["Wr"], d["W_gu"], d["W_d"], K, R)
    sel_ref = O.importance_topk(sc["g"], k)
    overlap = np.intersect1d(sel_gpu, sel_ref).size
    assert k - overlap <= 2, f"selection overlap {overlap}/{k}"
    # identical gradient -> identical selection
    sel_same = npu32(topk(torch.from_numpy(sc["g"].astype(np.float32)).to(DEV), k))
    assert np.array_equal(sel_same, sel_ref)
    # three steps on the oracle's selection
    lay.set_active(sel_ref)
    st = dict(W_gu=d["W_gu"], W_d=d["W_d"], Wr=d["Wr"], m=np.zeros(k), v=np.zeros(k),
              mr=np.zeros_like(d["Wr"]), vr=np.zeros_like(d["Wr"]), t=0)
    for step in range(3):
        lay.train_step(lr=1e-3)
        out = O.train_step(d["X"], d["tgt"], st["Wr"], st["W_gu"], st["W_d"], K, sel_ref,
                           st["m"], st["v"], st["mr"], st["vr"], st["t"], 1e-3, 0.9, 0.999,
                           1e-8, R)
        gu, dd = O.unflatten(out["W_flat"], shape)
        st.update(W_gu=gu, W_d=dd, Wr=out["Wr"], m=out["m"], v=out["v"], mr=out["mr"],
                  vr=out["vr"], t=out["t"])
        torch.cuda.synchronize()
        assert abs(float(lay.loss.item()) - out["loss"]) <= TOL_F32 * out["loss"]
    assert lay.t == 3
    flat = np.concatenate([st["W_gu"].ravel(), st["W_d"].ravel()])
    assert rel(npf(lay.W), flat) <= TOL_F32
    assert rel(npf(lay.m), st["m"]) <= TOL_F32
    assert rel(npf(lay.v), st["v"]) <= TOL_F32
    assert rel(npf(lay.Wr), st["Wr"]) <= TOL_F32
    assert rel(npf(lay.mr), st["mr"]) <= TOL_F32
    assert rel(npf(lay.vr), st["vr"]) <= TOL_F32


# --------------------------------------------------------------------------
# the pages' 4-bit storage, dequantised as the GEMMs load it
# --------------------------------------------------------------------------
def test_forward_q4_edge_scales_and_zeros(capi):
    """The 4-bit forward converts a row by one fused multiply-add only where
    that is exact (scale > 0 finite, zero 0 or |zero| >= 2^-10), otherwise as
    fp32(fp32(q - z) s): rows with negative, zero and subnormal scales, tiny,
    negative-zero, integer (q == z: exact zeros) and negative zeros, and zeros
    on both sides of 2^-10, give the same bits as the resident dequant (which
    equals the oracle's), in both weight tensors."""
    from sparse_fine_tuning_amd.layer import SparseMoELayer
    dims, group = (200, 256, 8, 2, 128), 64
    T, H, E, K, I = dims
    say(f"forward q4 edge scales dims={dims}")
    d = synth.moe_layer(*dims, bf16=True, seeds=(95, 96, 97, 98, 99))
    qg, sg, zg = synth.quantize_affine_int4(d["W_gu"].reshape(E * 2 * I, H), group)
    qd, sd, zd = synth.quantize_affine_int4(d["W_d"].reshape(E * H, I), group)
    edge = [(-0.5, None), (0.0, None), (2.0 ** -24, None), (0.25, 2.0 ** -12), (0.25, -0.0),
            (0.125, 3.0), (0.125, -2.5), (0.0625, 2.0 ** -10), (0.0625, 2.0 ** -11),
            (-0.25, 7.0), (0.5, 15.0)]
    for sarr, zarr in ((sg, zg), (sd, zd)):
        for i, (sv, zv) in enumerate(edge):
            for row in (i, 37 + 5 * i, sarr.shape[0] - 1 - i):  # rows in several tiles and waves
                sarr[row] = np.float16(sv).view(np.uint16)  # the arrays hold fp16 bits
                if zv is not None:
                    zarr[row] = np.float16(zv).view(np.uint16)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    i16 = lambda a: dev(np.ascontiguousarray(a).view(np.int16))
    tq = [dev(qg), i16(sg), i16(zg), dev(qd), i16(sd), i16(zd)]
    res = SparseMoELayer(*dims, act=capi.BF16, device=DEV)
    res.load(d["X"], d["Wr"], np.zeros_like(d["W_gu"]), np.zeros_like(d["W_d"]), d["tgt"])
    ngu = E * 2 * I * H
    capi.dequant_affine(tq[0], tq[1], tq[2], E * 2 * I, H, group, res.W[:ngu])
    capi.dequant_affine(tq[3], tq[4], tq[5], E * H, I, group, res.W[ngu:])
    res.forward()
    onl = SparseMoELayer(*dims, act=capi.BF16, device=DEV)
    onl.X, onl.Wr = res.X, res.Wr
    capi.moe_forward_q4(onl.shape, onl.X, onl.Wr, capi.q4_experts(*tq, group), onl.Y, onl.state,
                        onl.ws_fwd)
    torch.cuda.synchronize()
    for name in ("gu", "a"):
        assert torch.equal(res.st[name].view(torch.int16), onl.st[name].view(torch.int16)), name
    assert torch.equal(res.Y.view(torch.int16), onl.Y.view(torch.int16))
    W_gu = O.dequant_affine(qg, sg, zg, group)
    W_d = O.dequant_affine(qd, sd, zd, group)
    assert np.array_equal(bf16_bits(W_gu.ravel()),
                          res.W[:ngu].view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(bf16_bits(W_d.ravel()),
                          res.W[ngu:].view(torch.int16).cpu().numpy().view(np.uint16))


# (1, 256, 8, 2, 128) and (8, 256, 16, 1, 128): most experts empty;
# (1024, 256, 4, 2, 128): 512 slots per expert on average, the 256-row tiles
# (2200, 4096, 4, 2, 256) and (2000, 2048, 24, 4, 256): down launches whose
# last round is split in 2 and 4 contraction parts (a part may start on the
# second group of a scale pair); (1024, 2048, 16, 4, 1152): gate_up split in 4
@pytest.mark.parametrize("dims,group", [((1, 256, 8, 2, 128), 64), ((8, 256, 16, 1, 128), 64),
                                        ((200, 256, 8, 2, 128), 64), ((333, 512, 16, 4, 384), 64),
                                        ((1024, 256, 4, 2, 128), 64),
                                        ((1024, 2048, 128, 8, 768), 128),
                                        ((2200, 4096, 4, 2, 256), 64),
                                        ((2000, 2048, 24, 4, 256), 128),
                                        ((1024, 2048, 16, 4, 1152), 64)])
def test_forward_q4_equals_resident_dequant(capi, dims, group):
    """usaf_moe_forward_q4 on affine 4-bit codes against usaf_moe_forward on
    the usaf_dequant_affine copy of the same codes: every state tensor and
    the output bit-identical; and against the oracle's layer on the oracle's
    dequant of the codes within the bf16 tolerance (routing exact up to
    near-ties)."""
    from sparse_fine_tuning_amd.layer import SparseMoELayer
    T, H, E, K, I = dims
    say(f"forward q4 dims={dims} group={group}")
    d = synth.moe_layer(*dims, bf16=True, seeds=(90, 91, 92, 93, 94))
    qg, sg, zg = synth.quantize_affine_int4(d["W_gu"].reshape(E * 2 * I, H), group)
    qd, sd, zd = synth.quantize_affine_int4(d["W_d"].reshape(E * H, I), group)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    i16 = lambda a: dev(np.ascontiguousarray(a).view(np.int16))
    tq = [dev(qg), i16(sg), i16(zg), dev(qd), i16(sd), i16(zd)]
    # resident: dequantise into the flat weights, then the usual forward
    res = SparseMoELayer(*dims, act=capi.BF16, device=DEV)
    res.load(d["X"], d["Wr"], np.zeros_like(d["W_gu"]), np.zeros_like(d["W_d"]), d["tgt"])
    ngu = E * 2 * I * H
    capi.dequant_affine(tq[0], tq[1], tq[2], E * 2 * I, H, group, res.W[:ngu])
    capi.dequant_affine(tq[3], tq[4], tq[5], E * H, I, group, res.W[ngu:])
    res.forward()
    # on load: the same codes, no resident copy
    onl = SparseMoELayer(*dims, act=capi.BF16, device=DEV)
    onl.X, onl.Wr = res.X, res.Wr
    capi.moe_forward_q4(onl.shape, onl.X, onl.Wr, capi.q4_experts(*tq, group), onl.Y, onl.state,
                        onl.ws_fwd)
    torch.cuda.synchronize()
    for name in ("logits", "topk_ids", "topk_w", "offsets", "perm", "slot_pos", "gu", "a"):
        x, y = res.st[name], onl.st[name]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), name
    assert torch.equal(res.Y.view(torch.int16), onl.Y.view(torch.int16))
    split_cases = ((2200, 4096, 4, 2, 256), (2000, 2048, 24, 4, 256), (1024, 2048, 16, 4, 1152))
    if dims in split_cases and torch.cuda.get_device_properties(0).multi_processor_count == 256:
        off = res.st["offsets"].cpu().numpy()
        parts = {g: tail_split_parts(off, dims, g) for g in ("gate_up", "down")}
        say(f"  tail split parts: {parts}")
        assert max(parts.values()) >= 2, "the case no longer exercises the tail split"
    # the oracle: its dequant of the codes, then its layer
    R = O.Rounding(O.BF16, O.CONTRACT)
    W_gu = O.dequant_affine(qg, sg, zg, group).reshape(E, 2 * I, H)
    W_d = O.dequant_affine(qd, sd, zd, group).reshape(E, H, I)
    assert np.array_equal(bf16_bits(W_gu.ravel()),
                          res.W[:ngu].view(torch.int16).cpu().numpy().view(np.uint16))
    fw = O.moe_forward(d["X"], d["Wr"], W_gu, W_d, K, R)
    ids = onl.st["topk_ids"].cpu().numpy()
    logits = fw["logits"]
    bad = np.nonzero(np.any(ids != fw["topk_ids"], axis=1))[0]
    for t in bad:  # a routing difference must be a near-tie of the oracle's logits
        srt = np.sort(logits[t])[::-1]
        assert srt[K - 1] - srt[K] <= 1e-5 * np.abs(logits).max()
    ok = np.ones(T, bool)
    ok[bad] = False
    assert rel(npf(onl.Y)[ok], fw["Y"][ok]) <= TOL_BF16

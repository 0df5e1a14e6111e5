"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/usaf.h declares, sizes workspaces, and refuses bad arguments
before touching the device."""
import ctypes as C
import os
import re

import pytest

from sparse_fine_tuning_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "usaf.h")


def declared_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"USAF_API\s+[\w\s\*]+?\b(usaf_\w+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) >= 11
    lib = C.CDLL(capi.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(capi.EXPORTS)


def test_status_strings_and_version():
    assert capi.status_string(0) == "ok"
    assert "workspace" in capi.status_string(3)
    assert capi.status_string(99) == "unknown status"
    assert capi.version() >= 100


QWEN = capi.Shape(4096, 2048, 128, 8, 768, capi.BF16)


def test_workspace_sizes():
    S, H = QWEN.T * QWEN.K, QWEN.H
    assert capi.workspace_size(capi.WS_FORWARD, QWEN) >= S * H * 4
    assert capi.workspace_size(capi.WS_BACKWARD, QWEN) >= S * H * 4 + S * 4
    n = QWEN.N
    assert capi.workspace_size(capi.WS_TOPK, None, n) >= 2 * (n // 4096) * 4
    assert capi.workspace_size(capi.WS_RIGL, None, n, 3019898) >= 3 * 3019898 * 4


@pytest.mark.parametrize("shape,status", [
    (capi.Shape(0, 64, 8, 2, 32, 0), capi.USAF_ERR_INVALID_ARG),
    (capi.Shape(8, 64, 2, 3, 32, 0), capi.USAF_ERR_INVALID_ARG),     # K > E
    (capi.Shape(8, 64, 8, 2, 32, 7), capi.USAF_ERR_INVALID_ARG),     # bad dtype
    (capi.Shape(8, 60, 8, 2, 32, 0), capi.USAF_ERR_UNSUPPORTED),     # H % 64
    (capi.Shape(8, 64, 8, 2, 48, 0), capi.USAF_ERR_UNSUPPORTED),     # I % 32
    (capi.Shape(8, 64, 2048, 2, 32, 0), capi.USAF_ERR_UNSUPPORTED),  # E > 1024
    (capi.Shape(8, 8192, 128, 8, 8192, 1), capi.USAF_ERR_UNSUPPORTED),  # N >= 2^32
])
def test_shape_validation(shape, status):
    out = C.c_size_t(0)
    assert capi.lib.usaf_workspace_size(capi.WS_FORWARD, C.byref(shape), 0, 0, C.byref(out)) == status


def test_bad_workspace_kind_and_sizes():
    out = C.c_size_t(0)
    assert capi.lib.usaf_workspace_size(9, None, 0, 0, C.byref(out)) == capi.USAF_ERR_INVALID_ARG
    assert capi.lib.usaf_workspace_size(capi.WS_TOPK, None, -1, 0, C.byref(out)) == capi.USAF_ERR_INVALID_ARG
    assert capi.lib.usaf_workspace_size(capi.WS_TOPK, None, 2 ** 32, 0, C.byref(out)) == capi.USAF_ERR_INVALID_ARG
    assert capi.lib.usaf_workspace_size(capi.WS_RIGL, None, 10, 11, C.byref(out)) == capi.USAF_ERR_INVALID_ARG
    assert capi.lib.usaf_workspace_size(capi.WS_TOPK, None, 10, 0, None) == capi.USAF_ERR_INVALID_ARG


FAKE = 0x1000  # never dereferenced: every call below fails validation first


def test_entry_points_refuse_bad_arguments_before_launch():
    L = capi.lib
    sh = capi.Shape(128, 64, 8, 2, 32, 0)
    st = capi.State(*([FAKE] * 10))
    # forward: null input, missing workspace
    assert L.usaf_moe_forward(C.byref(sh), None, FAKE, FAKE, FAKE, C.byref(st), FAKE, 1 << 30, None) == 1
    assert L.usaf_moe_forward(C.byref(sh), FAKE, FAKE, FAKE, FAKE, C.byref(st), None, 0, None) == 3
    assert L.usaf_moe_forward(C.byref(sh), FAKE, FAKE, FAKE, FAKE, C.byref(st), FAKE, 16, None) == 3
    bad_state = capi.State(*([FAKE] * 9 + [0]))
    # backward: dense mode needs nnz == N; nnz range; state needs dgu/dw
    N = sh.N
    assert L.usaf_masked_backward(C.byref(sh), FAKE, FAKE, FAKE, C.byref(st), FAKE, None, N - 1,
                                  None, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert L.usaf_masked_backward(C.byref(sh), FAKE, FAKE, FAKE, C.byref(st), FAKE, FAKE, N + 1,
                                  None, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert L.usaf_masked_backward(C.byref(sh), FAKE, FAKE, FAKE, C.byref(bad_state), FAKE, FAKE, 5,
                                  None, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == 1
    # a sparse list on a bf16 layer whose X reaches 4 GiB (T*H*2 = 2^32 bytes):
    # the masked gradient addresses operand rows by 32-bit offsets
    big = capi.Shape(1 << 20, 2048, 8, 2, 32, 1)
    assert L.usaf_masked_backward(C.byref(big), FAKE, FAKE, FAKE, C.byref(st), FAKE, FAKE, 5,
                                  None, FAKE, FAKE, None, None, FAKE, 1 << 62, None) == 2
    # masked plan: nnz range, a list pointer, the plan's size (bf16 layers)
    shb = capi.Shape(128, 64, 8, 2, 32, 1)
    need = capi.workspace_size(capi.WS_MASKED_PLAN, shb)
    assert L.usaf_masked_plan(C.byref(shb), FAKE, -1, FAKE, need, None) == 1
    assert L.usaf_masked_plan(C.byref(shb), FAKE, N + 1, FAKE, need, None) == 1
    assert L.usaf_masked_plan(C.byref(shb), None, 5, FAKE, need, None) == 1
    assert L.usaf_masked_plan(C.byref(shb), FAKE, 5, FAKE, need - 1, None) == 3
    assert L.usaf_masked_plan(C.byref(shb), FAKE, 5, None, need, None) == 3
    assert L.usaf_masked_plan(C.byref(shb), None, 0, FAKE, need, None) == 0  # empty list: nothing to plan
    # 4-bit forward: fp32 layers, a group other than 64 / 128, misaligned codes or scales, nulls
    shq = capi.Shape(128, 256, 8, 2, 128, 1)
    q4 = lambda group=64, q=FAKE, sc=FAKE: capi.Q4Experts(q, sc, FAKE, q, sc, FAKE, group)
    fwd_q4 = lambda shape, w: L.usaf_moe_forward_q4(C.byref(shape), FAKE, FAKE, C.byref(w), FAKE,
                                                   C.byref(st), FAKE, 1 << 30, None)
    assert fwd_q4(capi.Shape(128, 256, 8, 2, 128, 0), q4()) == 2
    assert fwd_q4(shq, q4(group=32)) == 2
    assert fwd_q4(shq, q4(q=FAKE + 4)) == 2
    assert fwd_q4(shq, q4(sc=FAKE + 2)) == 2
    assert fwd_q4(shq, q4(q=0)) == 1
    assert fwd_q4(capi.Shape(128, 256, 8, 2, 192, 1), q4()) == 2  # I / 64 = 3 groups: odd
    assert L.usaf_masked_plan(C.byref(sh), FAKE, 5, None, 0, None) == 0      # fp32 layers need no plan
    # top-k: k larger than the candidates; k == 0 is a no-op
    assert L.usaf_importance_topk(FAKE, 100, 101, None, 0, FAKE, None, FAKE, 1 << 20, None) == 1
    assert L.usaf_importance_topk(FAKE, 100, 91, FAKE, 10, FAKE, None, FAKE, 1 << 20, None) == 1
    assert L.usaf_importance_topk(FAKE, 100, 0, None, 0, None, None, None, 0, None) == 0
    assert L.usaf_importance_topk(FAKE, 100, 5, None, 0, FAKE, None, FAKE, 8, None) == 3
    # a workspace off 16-byte alignment
    assert L.usaf_importance_topk(FAKE, 100, 5, None, 0, FAKE, None, FAKE + 4, 1 << 20, None) == 2
    # rigl: r > k, k > N
    assert L.usaf_rigl_reselect(C.byref(sh), FAKE, FAKE, None, FAKE, FAKE, FAKE, 10, 11, FAKE, FAKE,
                                FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert L.usaf_rigl_reselect(C.byref(sh), FAKE, FAKE, None, FAKE, FAKE, FAKE, N + 1, 1, FAKE, FAKE,
                                FAKE, None, None, FAKE, 1 << 30, None) == 1
    # new_w needs old_w (the kept entries' weights come from it)
    assert L.usaf_rigl_reselect(C.byref(sh), FAKE, FAKE, None, FAKE, FAKE, FAKE, 10, 3, FAKE, FAKE,
                                FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert L.usaf_rigl_reselect(C.byref(sh), FAKE, FAKE, None, FAKE, FAKE, FAKE, 10, 3, FAKE, FAKE,
                                FAKE, None, None, FAKE + 4, 1 << 40, None) == 2
    # adam: step < 1, bad dtype, n == 0 no-op
    f = C.c_double
    assert L.usaf_sparse_adam(1, FAKE, None, 10, None, FAKE, FAKE, FAKE, 0, f(1e-3), f(.9), f(.999), f(1e-8), None, None) == 1
    assert L.usaf_sparse_adam(5, FAKE, None, 10, None, FAKE, FAKE, FAKE, 1, f(1e-3), f(.9), f(.999), f(1e-8), None, None) == 1
    assert L.usaf_sparse_adam(1, None, None, 0, None, None, None, None, 1, f(1e-3), f(.9), f(.999), f(1e-8), None, None) == 0
    # a compact weight list needs the index list
    assert L.usaf_sparse_adam(1, FAKE, None, 10, FAKE, FAKE, FAKE, FAKE, 1, f(1e-3), f(.9), f(.999), f(1e-8), None, None) == 1
    assert L.usaf_gather(7, FAKE, FAKE, 10, FAKE, None) == 1
    assert L.usaf_gather(1, None, None, 0, None, None) == 0
    assert L.usaf_scatter(7, FAKE, FAKE, 10, FAKE, None) == 1
    assert L.usaf_scatter(1, FAKE, None, 10, FAKE, None) == 1
    assert L.usaf_scatter(1, FAKE, FAKE, -1, FAKE, None) == 1
    assert L.usaf_scatter(1, None, None, 0, None, None) == 0
    # dequant: group != 64, cols % 64, negative rows, misaligned output
    assert L.usaf_dequant_resident(FAKE, FAKE, 4, 128, 128, FAKE, None) == 2
    assert L.usaf_dequant_resident(FAKE, FAKE, 4, 96, 64, FAKE, None) == 2
    assert L.usaf_dequant_resident(FAKE, FAKE, -1, 128, 64, FAKE, None) == 1
    # affine dequant: group not 64 / 128, cols % group, negative rows, null zero
    assert L.usaf_dequant_affine(FAKE, FAKE, FAKE, 4, 256, 32, FAKE, None) == 2
    assert L.usaf_dequant_affine(FAKE, FAKE, FAKE, 4, 192, 128, FAKE, None) == 2
    assert L.usaf_dequant_affine(FAKE, FAKE, FAKE, -1, 128, 128, FAKE, None) == 1
    assert L.usaf_dequant_affine(FAKE, FAKE, None, 4, 128, 128, FAKE, None) == 1
    assert L.usaf_dequant_affine(None, None, None, 0, 128, 128, None, None) == 0
    assert L.usaf_dequant_resident(FAKE, FAKE, 4, 128, 64, FAKE + 8, None) == 2
    # mse / route: nulls
    assert L.usaf_mse_grad(C.byref(sh), None, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == 1
    assert L.usaf_route(C.byref(sh), None, C.byref(st), None) == 1
    # the no-allocation loss: nulls, and inputs beyond its fixed scratch (2^28 elements)
    assert L.usaf_mse_grad_noalloc(C.byref(sh), None, FAKE, FAKE, FAKE, None, None) == 1
    big = capi.Shape(65536, 8192, 8, 2, 32, 1)
    assert L.usaf_mse_grad_noalloc(C.byref(big), FAKE, FAKE, FAKE, FAKE, None, None) == 2

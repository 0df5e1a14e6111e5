"""ctypes binding of libusaf.so (include/usaf.h): argument marshalling only.

Every function takes torch tensors (device memory) or None for nullable
pointers, passes their addresses and the current (or given) stream to the
C ABI, and raises UsafError on a non-OK status.  No arithmetic of the method
happens here; if the library is missing the import fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libusaf.so")

USAF_OK, USAF_ERR_INVALID_ARG, USAF_ERR_UNSUPPORTED, USAF_ERR_WORKSPACE, USAF_ERR_HIP, \
    USAF_ERR_NOT_IMPLEMENTED = range(6)
F32, BF16 = 0, 1
WS_FORWARD, WS_BACKWARD, WS_TOPK, WS_RIGL, WS_MASKED_PLAN, WS_UNION = range(6)

# Every symbol include/usaf.h declares.
EXPORTS = (
    "usaf_workspace_size", "usaf_moe_forward", "usaf_masked_backward", "usaf_importance_topk",
    "usaf_rigl_reselect", "usaf_sparse_adam", "usaf_dequant_resident", "usaf_dequant_affine",
    "usaf_mse_grad", "usaf_mse_grad_noalloc",
    "usaf_route", "usaf_status_string", "usaf_version", "usaf_timer_arm", "usaf_timer_read",
    "usaf_gather", "usaf_scatter", "usaf_residual_add", "usaf_masked_plan", "usaf_sorted_union",
    "usaf_adjacent_diff", "usaf_moe_forward_q4",
)

# Kernel classes of the timing hook (usaf_kernel_class).
K_ROUTER_GEMM, K_ROUTE, K_GATE_UP, K_DOWN, K_COMBINE_Y, K_DA, K_ROUTER_BWD, K_DX, K_COMBINE_DX, \
    K_MASKED_DW, K_DENSE_DW, K_MSE, K_ADAM, K_DEQUANT, K_TOPK, K_RIGL_MERGE = range(16)
KERNEL_CLASS_NAMES = ("router_gemm", "route", "gate_up", "down", "combine_y", "da",
                      "router_bwd", "dx", "combine_dx", "masked_dw", "dense_dw", "mse", "adam",
                      "dequant", "topk", "rigl_merge")


class UsafError(RuntimeError):
    def __init__(self, status: int, call: str):
        super().__init__(f"{call}: {status_string(status)} (status {status})")
        self.status = status


class Shape(C.Structure):
    _fields_ = [("T", C.c_int32), ("H", C.c_int32), ("E", C.c_int32), ("K", C.c_int32),
                ("I", C.c_int32), ("act", C.c_int32)]

    @property
    def S(self):
        return self.T * self.K

    @property
    def N(self):
        return 3 * self.E * self.H * self.I

    @property
    def n_gate_up(self):
        return 2 * self.E * self.I * self.H

    def __repr__(self):
        return f"Shape(T={self.T}, H={self.H}, E={self.E}, K={self.K}, I={self.I}, act={self.act})"


class State(C.Structure):
    _fields_ = [("logits", C.c_void_p), ("topk_ids", C.c_void_p), ("topk_w", C.c_void_p),
                ("offsets", C.c_void_p), ("perm", C.c_void_p), ("slot_pos", C.c_void_p),
                ("gu", C.c_void_p), ("a", C.c_void_p), ("dgu", C.c_void_p), ("dw", C.c_void_p)]


class Q4Experts(C.Structure):
    _fields_ = [("q_gu", C.c_void_p), ("s_gu", C.c_void_p), ("z_gu", C.c_void_p),
                ("q_d", C.c_void_p), ("s_d", C.c_void_p), ("z_d", C.c_void_p),
                ("group", C.c_int32)]


class RiglStats(C.Structure):
    _fields_ = [("n_drop", C.c_int64), ("n_grow", C.c_int64), ("topk_new_vs_old", C.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_fine_tuning_amd.build`")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "usaf_workspace_size": [i32, vp, i64, i64, C.POINTER(sz)],
        "usaf_moe_forward": [vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "usaf_moe_forward_q4": [vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "usaf_masked_backward": [vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp],
        "usaf_masked_plan": [vp, vp, i64, vp, sz, vp],
        "usaf_importance_topk": [vp, i64, i64, vp, i64, vp, vp, vp, sz, vp],
        "usaf_rigl_reselect": [vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp],
        "usaf_sparse_adam": [i32, vp, vp, i64, vp, vp, vp, vp, i64, C.c_double, C.c_double,
                             C.c_double, C.c_double, vp, vp],
        "usaf_gather": [i32, vp, vp, i64, vp, vp],
        "usaf_scatter": [i32, vp, vp, i64, vp, vp],
        "usaf_dequant_resident": [vp, vp, i64, i64, i32, vp, vp],
        "usaf_dequant_affine": [vp, vp, vp, i64, i64, i32, vp, vp],
        "usaf_mse_grad": [vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "usaf_mse_grad_noalloc": [vp, vp, vp, vp, vp, vp, vp],
        "usaf_route": [vp, vp, vp, vp],
        "usaf_residual_add": [i32, vp, vp, vp, i64, vp],
        "usaf_sorted_union": [vp, i64, vp, i64, vp, vp, vp, sz, vp],
        "usaf_adjacent_diff": [vp, i64, vp, vp],
        "usaf_status_string": [i32],
        "usaf_version": [],
        "usaf_timer_arm": [i32, i32],
        "usaf_timer_read": [vp, i32, C.POINTER(i32)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = C.c_int32
    lib.usaf_status_string.restype = C.c_char_p
    return lib


lib = _load()


def status_string(s: int) -> str:
    return lib.usaf_status_string(int(s)).decode()


def version() -> int:
    return int(lib.usaf_version())


def _p(t):
    """Address of a tensor (or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, call: str):
    if status != USAF_OK:
        raise UsafError(status, call)


def _shape_ref(shape):
    return C.byref(shape) if shape is not None else None


def workspace_size(kind: int, shape: Shape | None = None, n: int = 0, k: int = 0) -> int:
    out = C.c_size_t(0)
    _check(lib.usaf_workspace_size(kind, _shape_ref(shape), n, k, C.byref(out)),
           "usaf_workspace_size")
    return int(out.value)


def make_state(d: dict) -> State:
    """State struct from a dict of tensors (keys as in usaf_moe_state)."""
    return State(*[_p(d.get(name)) for name, _ in State._fields_])


def moe_forward(shape, X, Wr, Wflat, Y, state: State, ws, stream=None):
    _check(lib.usaf_moe_forward(C.byref(shape), _p(X), _p(Wr), _p(Wflat), _p(Y), C.byref(state),
                                _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "usaf_moe_forward")


def q4_experts(q_gu, s_gu, z_gu, q_d, s_d, z_d, group) -> Q4Experts:
    """The 4-bit expert-weight struct from device tensors (codes uint8,
    scales and zeros as 16-bit fp16 bit patterns)."""
    return Q4Experts(_p(q_gu), _p(s_gu), _p(z_gu), _p(q_d), _p(s_d), _p(z_d), int(group))


def moe_forward_q4(shape, X, Wr, w: Q4Experts, Y, state: State, ws, stream=None):
    _check(lib.usaf_moe_forward_q4(C.byref(shape), _p(X), _p(Wr), C.byref(w), _p(Y),
                                   C.byref(state), _p(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)),
           "usaf_moe_forward_q4")


def masked_backward(shape, X, Wr, Wflat, state: State, dY, idx, nnz, dW, dWr, dX, nonfinite, ws,
                    stream=None, plan=None):
    _check(lib.usaf_masked_backward(C.byref(shape), _p(X), _p(Wr), _p(Wflat), C.byref(state),
                                    _p(dY), _p(idx), int(nnz), _p(plan), _p(dW), _p(dWr), _p(dX),
                                    _p(nonfinite), _p(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)),
           "usaf_masked_backward")


def masked_plan(shape, idx, nnz, plan, stream=None):
    _check(lib.usaf_masked_plan(C.byref(shape), _p(idx), int(nnz), _p(plan),
                                plan.numel() * plan.element_size(), _stream(stream)),
           "usaf_masked_plan")


def importance_topk(grad, n, k, exclude, n_exclude, out_idx, out_val, ws, stream=None):
    _check(lib.usaf_importance_topk(_p(grad), int(n), int(k), _p(exclude), int(n_exclude),
                                    _p(out_idx), _p(out_val), _p(ws),
                                    ws.numel() * ws.element_size() if ws is not None else 0,
                                    _stream(stream)),
           "usaf_importance_topk")


def rigl_reselect(shape, grad, Wflat, old_idx, old_m, old_v, k, r, new_idx, new_m, new_v, stats,
                  ws, stream=None, old_w=None, new_w=None):
    _check(lib.usaf_rigl_reselect(C.byref(shape), _p(grad), _p(Wflat), _p(old_w), _p(old_idx), _p(old_m),
                                  _p(old_v), int(k), int(r), _p(new_idx), _p(new_m), _p(new_v), _p(new_w),
                                  _p(stats), _p(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)),
           "usaf_rigl_reselect")


def sparse_adam(w_dtype, W, idx, n, g, m, v, step, lr, beta1, beta2, eps, skip=None, stream=None,
                w_list=None):
    _check(lib.usaf_sparse_adam(int(w_dtype), _p(W), _p(idx), int(n), _p(w_list), _p(g), _p(m),
                                _p(v), int(step), float(lr), float(beta1), float(beta2),
                                float(eps), _p(skip), _stream(stream)),
           "usaf_sparse_adam")


def gather(w_dtype, W, idx, n, out, stream=None):
    _check(lib.usaf_gather(int(w_dtype), _p(W), _p(idx), int(n), _p(out), _stream(stream)),
           "usaf_gather")


def scatter(w_dtype, W, idx, n, vals, stream=None):
    _check(lib.usaf_scatter(int(w_dtype), _p(W), _p(idx), int(n), _p(vals), _stream(stream)),
           "usaf_scatter")


def dequant_affine(q, scale_f16, zero_f16, rows, cols, group, out_bf16, stream=None):
    _check(lib.usaf_dequant_affine(_p(q), _p(scale_f16), _p(zero_f16), int(rows), int(cols),
                                   int(group), _p(out_bf16), _stream(stream)),
           "usaf_dequant_affine")


def dequant_resident(q, scale_f16, rows, cols, group, out_bf16, stream=None):
    _check(lib.usaf_dequant_resident(_p(q), _p(scale_f16), int(rows), int(cols), int(group),
                                     _p(out_bf16), _stream(stream)),
           "usaf_dequant_resident")


def mse_grad(shape, Y, tgt, dY, loss, nonfinite, ws, stream=None):
    _check(lib.usaf_mse_grad(C.byref(shape), _p(Y), _p(tgt), _p(dY), _p(loss), _p(nonfinite),
                             _p(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "usaf_mse_grad")


def mse_grad_noalloc(shape, Y, tgt, dY, loss, nonfinite, stream=None):
    _check(lib.usaf_mse_grad_noalloc(C.byref(shape), _p(Y), _p(tgt), _p(dY), _p(loss),
                                     _p(nonfinite), _stream(stream)),
           "usaf_mse_grad_noalloc")


def residual_add(act, a, b, out, n, stream=None):
    _check(lib.usaf_residual_add(int(act), _p(a), _p(b), _p(out), int(n), _stream(stream)),
           "usaf_residual_add")


def sorted_union(a, na, b, nb, out, n_out, ws, stream=None):
    _check(lib.usaf_sorted_union(_p(a), int(na), _p(b), int(nb), _p(out), _p(n_out), _p(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)),
           "usaf_sorted_union")


def adjacent_diff(inp, n, out, stream=None):
    _check(lib.usaf_adjacent_diff(_p(inp), int(n), _p(out), _stream(stream)), "usaf_adjacent_diff")


def route(shape, logits, state: State, stream=None):
    _check(lib.usaf_route(C.byref(shape), _p(logits), C.byref(state), _stream(stream)),
           "usaf_route")


def timer_arm(kernel_class: int, capacity: int = 1024):
    """Arm the event-timing hook for one kernel class (-1 disarms)."""
    _check(lib.usaf_timer_arm(int(kernel_class), int(capacity)), "usaf_timer_arm")


def timer_read(capacity: int = 1024):
    """Milliseconds of each recorded launch of the armed class (waits for them)."""
    buf = (C.c_float * max(1, capacity))()
    n = C.c_int32(0)
    _check(lib.usaf_timer_read(buf, int(capacity), C.byref(n)), "usaf_timer_read")
    return [float(buf[i]) for i in range(n.value)]

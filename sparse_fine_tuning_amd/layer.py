"""One MoE layer's sparse fine-tuning step driven through the C ABI.

PyTorch is used only to own device memory and to supply the stream; every
step of the method runs in libusaf.so's HIP kernels:

  usaf_moe_forward -> usaf_mse_grad -> usaf_masked_backward
  -> usaf_sparse_adam (experts, at the active list) -> usaf_sparse_adam (router, dense)

and, periodically, the dense scan (usaf_masked_backward in dense mode),
usaf_importance_topk and usaf_rigl_reselect (the usaf README's importance
phase and RigL reselection).
"""
from __future__ import annotations

import numpy as np
import torch

from . import capi
from .capi import BF16, F32


def _dt(act: int):
    return torch.bfloat16 if act == BF16 else torch.float32


class SparseMoELayer:
    """Device buffers of one layer plus the calls of one train step."""

    def __init__(self, T, H, E, K, I, act=BF16, device="cuda"):
        self.shape = capi.Shape(T, H, E, K, I, act)
        self.device = torch.device(device)
        self.act = act
        dt = _dt(act)
        dev = self.device
        S = T * K
        z = lambda *s, dtype=torch.float32: torch.empty(*s, dtype=dtype, device=dev)
        self.st = dict(
            logits=z(T, E), topk_ids=z(T, K, dtype=torch.int32), topk_w=z(T, K),
            offsets=z(E + 1, dtype=torch.int32), perm=z(S, dtype=torch.int32),
            slot_pos=z(S, dtype=torch.int32), gu=z(S, 2 * I, dtype=dt), a=z(S, I, dtype=dt),
            dgu=z(S, 2 * I, dtype=dt), dw=z(T, K))
        self.state = capi.make_state(self.st)
        self.ws_fwd = z(capi.workspace_size(capi.WS_FORWARD, self.shape), dtype=torch.uint8)
        self.ws_bwd = z(capi.workspace_size(capi.WS_BACKWARD, self.shape), dtype=torch.uint8)
        self.Y = z(T, H, dtype=dt)
        self.dY = z(T, H, dtype=dt)
        self.dX = z(T, H, dtype=dt)
        self.dWr = z(E, H)
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.nonfinite = torch.zeros(1, dtype=torch.int32, device=dev)
        self.idx = None
        self.X = self.Wr = self.W = self.tgt = None
        self.t = 0
        self.skipped = 0

    # ---- parameters and data -------------------------------------------------
    @property
    def W(self):
        """The flat expert weights [N] (act dtype)."""
        return self._W

    @W.setter
    def W(self, value):
        # SparseAdam reads the active weights from the compact list, so a new
        # weight buffer must refresh it (else the next update would write the
        # old active weights back); after writing into W in place, call
        # refresh_list() for the same reason
        self._W = value
        if value is not None and self.idx is not None:
            self.refresh_list()

    def load(self, X, Wr, W_gu, W_d, tgt):
        """Upload numpy inputs (values already representable in the act dtype)."""
        dt, dev = _dt(self.act), self.device
        self.X = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).to(dev).to(dt)
        self.tgt = torch.from_numpy(np.ascontiguousarray(tgt, dtype=np.float32)).to(dev).to(dt)
        self.Wr = torch.from_numpy(np.ascontiguousarray(Wr, dtype=np.float32)).to(dev)
        flat = np.concatenate([np.asarray(W_gu, np.float32).ravel(), np.asarray(W_d, np.float32).ravel()])
        self.W = torch.from_numpy(flat).to(dev).to(dt)
        self.mr = torch.zeros_like(self.Wr)
        self.vr = torch.zeros_like(self.Wr)

    def set_batch(self, X, tgt):
        dt, dev = _dt(self.act), self.device
        self.X.copy_(torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).to(dev).to(dt))
        self.tgt.copy_(torch.from_numpy(np.ascontiguousarray(tgt, dtype=np.float32)).to(dev).to(dt))

    def set_active(self, idx_u32: np.ndarray):
        """Active list (ascending uint32 flat indices) with fresh Adam moments."""
        idx = np.ascontiguousarray(idx_u32, dtype=np.uint32).view(np.int32)
        self.idx = torch.from_numpy(idx).to(self.device)
        k = idx.size
        self.m = torch.zeros(k, dtype=torch.float32, device=self.device)
        self.v = torch.zeros(k, dtype=torch.float32, device=self.device)
        self.dW = torch.empty(k, dtype=torch.float32, device=self.device)
        self.refresh_list()

    def refresh_list(self, w_list=None):
        """Per-list state rebuilt whenever the list changes: the compact copy
        of the active weights (W at idx) that SparseAdam reads instead of the
        scattered entries (gathered, unless the caller has it, as RigL's
        reselection does), and the masked gradient's plan."""
        k = self.idx.numel()
        if w_list is None:
            w_list = torch.empty(k, dtype=_dt(self.act), device=self.device)
            capi.gather(self.act, self.W, self.idx, k, w_list)
        self.w_list = w_list
        if getattr(self, "plan", None) is None:
            self.plan = torch.empty(capi.workspace_size(capi.WS_MASKED_PLAN, self.shape),
                                    dtype=torch.uint8, device=self.device)
        capi.masked_plan(self.shape, self.idx, k, self.plan)

    # ---- the step ------------------------------------------------------------
    def forward(self, stream=None):
        capi.moe_forward(self.shape, self.X, self.Wr, self.W, self.Y, self.state, self.ws_fwd,
                         stream)

    def loss_grad(self, stream=None):
        capi.mse_grad(self.shape, self.Y, self.tgt, self.dY, self.loss, self.nonfinite,
                      self.ws_fwd, stream)

    def backward(self, dense_out=None, want_dx=True, stream=None):
        if dense_out is not None:
            capi.masked_backward(self.shape, self.X, self.Wr, self.W, self.state, self.dY, None,
                                 self.shape.N, dense_out, self.dWr, self.dX if want_dx else None,
                                 None, self.ws_bwd, stream)
        else:
            capi.masked_backward(self.shape, self.X, self.Wr, self.W, self.state, self.dY,
                                 self.idx, self.idx.numel(), self.dW, self.dWr,
                                 self.dX if want_dx else None, self.nonfinite, self.ws_bwd,
                                 stream, plan=self.plan)

    def adam(self, step, lr, betas=(0.9, 0.999), eps=1e-8, stream=None):
        b1, b2 = betas
        capi.sparse_adam(self.act, self.W, self.idx, self.idx.numel(), self.dW, self.m, self.v,
                         step, lr, b1, b2, eps, self.nonfinite, stream, w_list=self.w_list)
        capi.sparse_adam(F32, self.Wr, None, self.Wr.numel(), self.dWr, self.mr, self.vr, step,
                         lr, b1, b2, eps, self.nonfinite, stream)

    def train_step(self, lr, betas=(0.9, 0.999), eps=1e-8, stream=None, check_skip=True):
        """forward, loss, masked backward, SparseAdam (experts) + Adam (router).
        The step count advances only when the step was not skipped; checking
        that needs one 4-byte device->host read (check_skip=False avoids it
        and assumes a finite step)."""
        self.nonfinite.zero_()
        self.forward(stream)
        self.loss_grad(stream)
        self.backward(stream=stream)
        self.adam(self.t + 1, lr, betas, eps, stream)
        if check_skip and int(self.nonfinite.item()) != 0:
            self.skipped += 1
        else:
            self.t += 1

    # ---- importance / RigL ---------------------------------------------------
    def dense_scan(self, out=None, stream=None):
        """Forward, loss and the gradient of every expert weight (fp32 [N])."""
        if out is None:
            out = torch.empty(self.shape.N, dtype=torch.float32, device=self.device)
        self.forward(stream)
        self.loss_grad(stream)
        self.backward(dense_out=out, want_dx=False, stream=stream)
        return out


def topk(grad: torch.Tensor, k: int, exclude: torch.Tensor | None = None, stream=None,
         ws: torch.Tensor | None = None) -> torch.Tensor:
    """Ascending indices (int32 tensor holding uint32 values) of the top-k |grad|."""
    n = grad.numel()
    if ws is None:
        ws = torch.empty(capi.workspace_size(capi.WS_TOPK, None, n), dtype=torch.uint8,
                         device=grad.device)
    out = torch.empty(k, dtype=torch.int32, device=grad.device)
    nex = 0 if exclude is None else exclude.numel()
    capi.importance_topk(grad, n, k, exclude, nex, out, None, ws, stream)
    return out


def rigl(layer: SparseMoELayer, grad: torch.Tensor, r: int, stream=None, ws=None):
    """RigL reselection of the layer's active set; returns device stats [3] int64."""
    k = layer.idx.numel()
    N = layer.shape.N
    if ws is None:
        ws = torch.empty(capi.workspace_size(capi.WS_RIGL, None, N, k), dtype=torch.uint8,
                         device=layer.device)
    new_idx = torch.empty_like(layer.idx)
    new_m = torch.empty_like(layer.m)
    new_v = torch.empty_like(layer.v)
    stats = torch.zeros(3, dtype=torch.int64, device=layer.device)
    new_w = torch.empty_like(layer.w_list)
    capi.rigl_reselect(layer.shape, grad, layer.W, layer.idx, layer.m, layer.v, k, r, new_idx,
                       new_m, new_v, stats, ws, stream, old_w=layer.w_list, new_w=new_w)
    layer.idx, layer.m, layer.v = new_idx, new_m, new_v
    layer.refresh_list(w_list=new_w)
    return stats

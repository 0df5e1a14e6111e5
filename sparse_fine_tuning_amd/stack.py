"""A stack of MoE layers trained sparsely through the C ABI: the trainer loop
around the layer step.

The usaf README trains the expert weights of a deep model's MoE layers
("how it works": native sparse fine-tuning with the router trained densely;
environment-variable table: STEPS, LR_PEAK with cosine decay, FRAC,
RESELECT_EVERY).  Here the stack keeps only the MoE layers, joined by a
residual stream:

  forward   X_{l+1} = round(X_l + Y_l)                      (usaf_residual_add)
  loss      MSE of X_L against the target                    (usaf_mse_grad)
  backward  G_l = round(G_{l+1} + dX_l), layer l's weight gradients taken
            against output gradient G_{l+1}                  (usaf_masked_backward)
  update    every layer's SparseAdam + router Adam, one shared step count,
            all skipped together when any gradient is non-finite

and the importance pass / RigL reselection scan the dense gradient of every
layer in one backward, selecting each layer's list from its own gradient
before the next layer's backward reuses the dense buffer.

Around the step (README environment-variable table: STEPS, RESELECT_EVERY,
TRAIN_FROM, the NaN-skip count of the results): the layers below
``train_from`` are frozen, as the README freezes the lower layers of a
model -- they run their forward only, since no trainable weight lies below
them, and hold no list, moments or gradient buffers; a checkpoint holds
what a resume needs on top of the base weights (every trained layer's list,
moments, router and its moments, the weights at every index ever selected,
the step and skip counts); and the expert load of the last forward is
readable per layer.

PyTorch only owns device memory; every step runs in libusaf.so's kernels.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import capi
from .capi import BF16, F32


def _dt(act: int):
    return torch.bfloat16 if act == BF16 else torch.float32


def cosine_lr(step: int, total: int, peak: float) -> float:
    """README cosine decay from LR_PEAK at step 0 towards 0 at ``total``."""
    return 0.5 * peak * (1.0 + math.cos(math.pi * step / total))


class _Layer:
    """Parameters, optimiser state and saved forward state of one layer.  A
    frozen layer keeps its own routing state (for the expert-load monitor)
    but shares the large saved activations with the other frozen layers and
    has no router moments or gradient."""

    def __init__(self, shape: capi.Shape, shared: dict, dev: torch.device, frozen: bool = False):
        T, H, E, K, I, act = shape.T, shape.H, shape.E, shape.K, shape.I, shape.act
        dt = _dt(act)
        S = T * K
        z = lambda *s, dtype=torch.float32: torch.empty(*s, dtype=dtype, device=dev)
        big = shared["frozen_acts"] if frozen else dict(gu=z(S, 2 * I, dtype=dt), a=z(S, I, dtype=dt))
        self.st = dict(
            logits=z(T, E), topk_ids=z(T, K, dtype=torch.int32), topk_w=z(T, K),
            offsets=z(E + 1, dtype=torch.int32), perm=z(S, dtype=torch.int32),
            slot_pos=z(S, dtype=torch.int32), gu=big["gu"], a=big["a"],
            dgu=shared["dgu"], dw=shared["dw"])
        self.state = capi.make_state(self.st)
        self.frozen = frozen
        self.q4 = None  # a frozen layer's 4-bit codes (capi.Q4Experts and its tensors), if any
        self.W = z(shape.N, dtype=dt)
        self.Wr = z(E, H)
        if frozen:
            self.mr = self.vr = self.dWr = None
        else:
            self.mr = torch.zeros(E, H, dtype=torch.float32, device=dev)
            self.vr = torch.zeros(E, H, dtype=torch.float32, device=dev)
            self.dWr = z(E, H)
        self.shape = shape
        self.idx = self.m = self.v = self.dW = self.w_list = self.plan = None
        self.touched = None  # int32 tensor of ascending uint32: every index selected so far

    def note_touched(self):
        """Adds the current list to the touched set (its weights may differ
        from the base weights from now on: RigL keeps the values of dropped
        entries): a sorted-union merge on the device; its length is read
        back (one small synchronisation, at reselections only)."""
        if self.touched is None:
            self.touched = self.idx.clone()
            return
        na, nb = self.touched.numel(), self.idx.numel()
        out = torch.empty(na + nb, dtype=torch.int32, device=self.idx.device)
        n_out = torch.zeros(1, dtype=torch.int64, device=self.idx.device)
        ws = torch.empty(capi.workspace_size(capi.WS_UNION, None, na + nb), dtype=torch.uint8,
                         device=self.idx.device)
        capi.sorted_union(self.touched, na, self.idx, nb, out, n_out, ws)
        self.touched = out[: int(n_out.item())].clone()

    def set_active(self, idx: torch.Tensor, act: int):
        """Active list (int32 tensor of ascending uint32 flat indices) with
        fresh moments."""
        k = idx.numel()
        dev = idx.device
        self.idx = idx
        self.m = torch.zeros(k, dtype=torch.float32, device=dev)
        self.v = torch.zeros(k, dtype=torch.float32, device=dev)
        self.dW = torch.empty(k, dtype=torch.float32, device=dev)
        self.note_touched()
        self.refresh_list(act)

    def refresh_list(self, act: int, w_list=None):
        """The compact weight list SparseAdam reads (gathered, unless the
        caller has it, as RigL's reselection does) and the masked gradient's
        plan, both rebuilt whenever the list changes."""
        k = self.idx.numel()
        if w_list is None:
            w_list = torch.empty(k, dtype=_dt(act), device=self.idx.device)
            capi.gather(act, self.W, self.idx, k, w_list)
        self.w_list = w_list
        if self.plan is None:
            self.plan = torch.empty(capi.workspace_size(capi.WS_MASKED_PLAN, self.shape),
                                    dtype=torch.uint8, device=self.idx.device)
        capi.masked_plan(self.shape, self.idx, k, self.plan)


class MoEStack:
    """``n_layers`` MoE layers of one shape on one device."""

    def __init__(self, n_layers, T, H, E, K, I, act=BF16, device="cuda", train_from=0):
        if not 0 <= train_from < n_layers:
            raise ValueError("train_from must name a layer of the stack")
        self.shape = capi.Shape(T, H, E, K, I, act)
        self.act = act
        self.n_layers = n_layers
        self.train_from = train_from
        self.device = dev = torch.device(device)
        dt = _dt(act)
        z = lambda *s, dtype=torch.float32: torch.empty(*s, dtype=dtype, device=dev)
        shared = dict(dgu=z(T * K, 2 * I, dtype=dt), dw=z(T, K))
        if train_from > 0:
            shared["frozen_acts"] = dict(gu=z(T * K, 2 * I, dtype=dt), a=z(T * K, I, dtype=dt))
        self.layers = [_Layer(self.shape, shared, dev, frozen=l < train_from)
                       for l in range(n_layers)]
        self.ws_fwd = z(capi.workspace_size(capi.WS_FORWARD, self.shape), dtype=torch.uint8)
        self.ws_bwd = z(capi.workspace_size(capi.WS_BACKWARD, self.shape), dtype=torch.uint8)
        self.Xs = [z(T, H, dtype=dt) for _ in range(n_layers + 1)]  # X_0 .. X_L
        self.tgt = z(T, H, dtype=dt)
        self.Y = z(T, H, dtype=dt)
        self.dXl = z(T, H, dtype=dt)
        self.G = [z(T, H, dtype=dt), z(T, H, dtype=dt)]
        self.loss = torch.zeros(1, dtype=torch.float32, device=dev)
        self.nonfinite = torch.zeros(1, dtype=torch.int32, device=dev)
        self.t = 0
        self.skipped = 0
        self._dense = None
        self._ws_topk = None
        self._ws_rigl = None

    # ---- parameters and data -----------------------------------------------
    def load_layer(self, l, W_gu, W_d, Wr):
        """Upload one layer's numpy weights (values representable in act)."""
        lay, dev, dt = self.layers[l], self.device, _dt(self.act)
        flat = np.concatenate([np.asarray(W_gu, np.float32).ravel(), np.asarray(W_d, np.float32).ravel()])
        lay.W.copy_(torch.from_numpy(flat).to(dev).to(dt))
        lay.Wr.copy_(torch.from_numpy(np.ascontiguousarray(Wr, dtype=np.float32)).to(dev))
        if lay.idx is not None:  # SparseAdam's compact copy of the active weights
            lay.refresh_list(self.act)

    def load_layer_q4(self, l, codes, group, Wr):
        """A frozen layer whose experts stay in the pages' 4-bit storage (the
        affine codes of usaf_dequant_affine: q_gu, s_gu, z_gu, q_d, s_d, z_d as
        numpy arrays, scales and zeros as fp16 bit patterns) and are
        dequantised as its forward loads them: no resident bf16 copy."""
        lay = self.layers[l]
        if not lay.frozen:
            raise ValueError("only frozen layers (below train_from) keep 4-bit experts")
        dev = self.device
        ts = [torch.from_numpy(np.ascontiguousarray(c).view(np.int16 if c.dtype == np.uint16 else c.dtype))
              .to(dev) for c in codes]
        lay.q4 = (capi.q4_experts(*ts, group), ts)
        lay.W = None  # the resident copy is not kept
        lay.Wr.copy_(torch.from_numpy(np.ascontiguousarray(Wr, dtype=np.float32)).to(dev))

    def set_batch(self, X, tgt):
        """X_0 and the target: numpy arrays or device tensors."""
        for dst, src in ((self.Xs[0], X), (self.tgt, tgt)):
            if isinstance(src, torch.Tensor):
                dst.copy_(src)
            else:
                dst.copy_(torch.from_numpy(np.ascontiguousarray(src, dtype=np.float32)).to(self.device))

    # ---- the step ------------------------------------------------------------
    def forward(self, stream=None):
        n = self.shape.T * self.shape.H
        for l, lay in enumerate(self.layers):
            if lay.q4 is not None:
                capi.moe_forward_q4(self.shape, self.Xs[l], lay.Wr, lay.q4[0], self.Y, lay.state,
                                    self.ws_fwd, stream)
            else:
                capi.moe_forward(self.shape, self.Xs[l], lay.Wr, lay.W, self.Y, lay.state,
                                 self.ws_fwd, stream)
            capi.residual_add(self.act, self.Xs[l], self.Y, self.Xs[l + 1], n, stream)

    def backward(self, select=None, stream=None):
        """Backward from the loss of the last output down to the lowest
        trained layer (nothing below it trains, so it forms no input
        gradient).  With ``select`` (a callable (l, dense_grad)), every
        trained layer's dense expert-weight gradient is formed instead of the
        listed one and handed to it at once."""
        n = self.shape.T * self.shape.H
        capi.mse_grad(self.shape, self.Xs[-1], self.tgt, self.G[0], self.loss, self.nonfinite,
                      self.ws_fwd, stream)
        cur = 0
        for l in range(self.n_layers - 1, self.train_from - 1, -1):
            lay = self.layers[l]
            G, Gn = self.G[cur], self.G[cur ^ 1]
            dX = self.dXl if l > self.train_from else None
            if select is None:
                capi.masked_backward(self.shape, self.Xs[l], lay.Wr, lay.W, lay.state, G, lay.idx,
                                     lay.idx.numel(), lay.dW, lay.dWr, dX, self.nonfinite,
                                     self.ws_bwd, stream, plan=lay.plan)
            else:
                dense = self._dense_buffer()
                capi.masked_backward(self.shape, self.Xs[l], lay.Wr, lay.W, lay.state, G, None,
                                     self.shape.N, dense, lay.dWr, dX, None, self.ws_bwd, stream)
                select(l, dense)
            if l > self.train_from:
                capi.residual_add(self.act, G, self.dXl, Gn, n, stream)
                cur ^= 1

    def trained(self):
        """The layers that train (from ``train_from`` up)."""
        return self.layers[self.train_from:]

    def adam(self, step, lr, betas=(0.9, 0.999), eps=1e-8, stream=None):
        b1, b2 = betas
        for lay in self.trained():
            capi.sparse_adam(self.act, lay.W, lay.idx, lay.idx.numel(), lay.dW, lay.m, lay.v, step,
                             lr, b1, b2, eps, self.nonfinite, stream, w_list=lay.w_list)
            capi.sparse_adam(F32, lay.Wr, None, lay.Wr.numel(), lay.dWr, lay.mr, lay.vr, step, lr,
                             b1, b2, eps, self.nonfinite, stream)

    def train_step(self, lr, betas=(0.9, 0.999), eps=1e-8, stream=None, check_skip=True):
        """Forward, loss, backward through every layer, then every layer's
        update with the shared step count (skipped together when any gradient
        is non-finite; checking that costs one 4-byte device->host read)."""
        self.nonfinite.zero_()
        self.forward(stream)
        self.backward(stream=stream)
        self.adam(self.t + 1, lr, betas, eps, stream)
        if check_skip and int(self.nonfinite.item()) != 0:
            self.skipped += 1
        else:
            self.t += 1

    # ---- importance / RigL ---------------------------------------------------
    def _dense_buffer(self):
        if self._dense is None:
            self._dense = torch.empty(self.shape.N, dtype=torch.float32, device=self.device)
        return self._dense

    def _topk_ws(self):
        if self._ws_topk is None:
            self._ws_topk = torch.empty(capi.workspace_size(capi.WS_TOPK, None, self.shape.N),
                                        dtype=torch.uint8, device=self.device)
        return self._ws_topk

    def importance(self, k: int, stream=None):
        """The importance pass: every trained layer's active list is the
        top-k of its own dense gradient on the current batch."""
        ws = self._topk_ws()

        def pick(l, grad):
            out = torch.empty(k, dtype=torch.int32, device=self.device)
            capi.importance_topk(grad, self.shape.N, k, None, 0, out, None, ws, stream)
            self.layers[l].set_active(out, self.act)

        self.forward(stream)
        self.backward(select=pick, stream=stream)

    def rigl(self, r: int, stream=None) -> torch.Tensor:
        """RigL reselection of every trained layer on the current batch;
        returns the device stats [n_layers, 3] (int64) of usaf_rigl_reselect
        (zero rows for frozen layers)."""
        k = self.layers[self.train_from].idx.numel()
        if self._ws_rigl is None:
            self._ws_rigl = torch.empty(capi.workspace_size(capi.WS_RIGL, None, self.shape.N, k),
                                        dtype=torch.uint8, device=self.device)
        stats = torch.zeros(self.n_layers, 3, dtype=torch.int64, device=self.device)

        def reselect(l, grad):
            lay = self.layers[l]
            new_idx = torch.empty_like(lay.idx)
            new_m = torch.empty_like(lay.m)
            new_v = torch.empty_like(lay.v)
            new_w = torch.empty_like(lay.w_list)
            capi.rigl_reselect(self.shape, grad, lay.W, lay.idx, lay.m, lay.v, k, r, new_idx,
                               new_m, new_v, stats[l], self._ws_rigl, stream, old_w=lay.w_list,
                               new_w=new_w)
            lay.idx, lay.m, lay.v = new_idx, new_m, new_v
            lay.note_touched()
            lay.refresh_list(self.act, w_list=new_w)

        self.forward(stream)
        self.backward(select=reselect, stream=stream)
        return stats

    # ---- monitoring, checkpoint / resume --------------------------------------
    def expert_load(self) -> torch.Tensor:
        """Slots routed to each expert in every layer's last forward: int32
        [n_layers, E] (each row sums to T*K), the differences of each layer's
        expert offsets."""
        E = self.shape.E
        out = torch.empty(self.n_layers, E, dtype=torch.int32, device=self.device)
        for l, lay in enumerate(self.layers):
            capi.adjacent_diff(lay.st["offsets"], E, out[l])
        return out

    def state_dict(self) -> dict:
        """Host tensors of a resume point: the step and skip counts and, per
        layer, the list, its moments, the router and its moments, and the
        touched indices with their current weights.  The weights outside the
        touched set are the base weights, which the resuming stack loads
        itself (a 48-layer Qwen3-shaped stack holds 58 GB of them)."""
        sd = {"t": torch.tensor([self.t], dtype=torch.int64),
              "skipped": torch.tensor([self.skipped], dtype=torch.int64),
              "train_from": torch.tensor([self.train_from], dtype=torch.int64)}
        for l, lay in enumerate(self.layers):
            if lay.frozen:
                continue
            p = f"layer{l}."
            sd[p + "idx"] = lay.idx.cpu()
            sd[p + "m"] = lay.m.cpu()
            sd[p + "v"] = lay.v.cpu()
            sd[p + "Wr"] = lay.Wr.cpu()
            sd[p + "mr"] = lay.mr.cpu()
            sd[p + "vr"] = lay.vr.cpu()
            sd[p + "touched"] = lay.touched.cpu()
            tw = torch.empty(lay.touched.numel(), dtype=lay.W.dtype, device=lay.W.device)
            capi.gather(self.act, lay.W, lay.touched, lay.touched.numel(), tw)
            sd[p + "touched_w"] = tw.cpu()
        return sd

    def load_state_dict(self, sd: dict):
        """Restores a resume point onto a stack of the same shape whose base
        weights are loaded; the following steps then repeat, bit for bit, the
        steps of the run that saved it."""
        dev = self.device
        if int(sd.get("train_from", torch.zeros(1, dtype=torch.int64))[0]) != self.train_from:
            raise ValueError("the checkpoint was saved by a stack with another train_from")
        self.t = int(sd["t"][0])
        self.skipped = int(sd["skipped"][0])
        for l, lay in enumerate(self.layers):
            if lay.frozen:
                continue
            p = f"layer{l}."
            touched = sd[p + "touched"].to(dev)
            tw = sd[p + "touched_w"].to(dev)
            if touched.numel() != tw.numel() or tw.dtype != lay.W.dtype:
                raise ValueError(f"layer {l}: touched weights do not match the touched list")
            capi.scatter(self.act, lay.W, touched, touched.numel(), tw)
            lay.Wr.copy_(sd[p + "Wr"].to(dev))
            lay.mr.copy_(sd[p + "mr"].to(dev))
            lay.vr.copy_(sd[p + "vr"].to(dev))
            lay.idx = sd[p + "idx"].to(dev).clone()
            lay.m = sd[p + "m"].to(dev).clone()
            lay.v = sd[p + "v"].to(dev).clone()
            lay.dW = torch.empty_like(lay.m)
            lay.touched = touched
            lay.refresh_list(self.act)

    def save(self, path: str):
        """The state dict as a safetensors file."""
        from safetensors.torch import save_file
        save_file(self.state_dict(), path)

    def load(self, path: str):
        from safetensors.torch import load_file
        self.load_state_dict(load_file(path))

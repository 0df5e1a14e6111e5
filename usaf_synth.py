"""Seeded synthetic inputs for the USAF sparse MoE layer.

This module is the only code shared by the CPU oracle (``oracle/``) and the HIP
path (``sparse_fine_tuning_amd``).  It draws random numbers and packs them into
the layouts the two sides consume; it contains none of the method's arithmetic
(no routing, no gradients, no optimiser, no selection).

The pages measure on real Qwen3-30B-A3B weights and a tokenised code dataset
(usaf README, intro and RX 6750 XT results table); neither is available, so
seeded Gaussian tensors of the same shapes stand in for them:

* activations X ~ N(0, 1), regression target ~ N(0, 1);
* expert weights and the router ~ N(0, 0.02);
* bf16 configurations hold bf16-representable values (rounded once, here, with
  torch's round-to-nearest-even conversion) so both sides see identical inputs;
* the fixed "active mask" is ``k`` distinct flat indices drawn uniformly and
  sorted ascending;
* the int4 resident-dequant input is produced by a plain symmetric quantiser
  (group of 64 along the input dim, fp16 scale = amax / 7, codes in [-7, 7]).

Weight layout (the fused expert tensors of the usaf README's quantisation
recipe): ``W_gu`` is ``[E, 2I, H]`` (rows ``[0, I)`` gate, ``[I, 2I)`` up) and
``W_d`` is ``[E, H, I]``; both are stored out x in.  The flat parameter vector
of one layer is ``concat(W_gu.ravel(), W_d.ravel())``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "normal", "to_bf16_values", "moe_layer", "random_mask", "quantize_int4_g64",
    "flat_weights", "SHAPES",
]

# Named layer shapes (T, H, E, K, I).
SHAPES = {
    "tiny_fp32": dict(T=128, H=64, E=8, K=2, I=32),
    "qwen3_30b_a3b": dict(T=4096, H=2048, E=128, K=8, I=768),
    "mixtral_8x7b": dict(T=4096, H=4096, E=8, K=2, I=14336),
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def normal(shape, sigma: float, seed: int) -> np.ndarray:
    """fp32 array of N(0, sigma^2) draws from PCG64(seed)."""
    z = _rng(seed).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        z *= np.float32(sigma)
    return z


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """fp32 array whose values are the bf16 round-to-nearest-even of ``x``.

    Uses torch's dtype conversion; this is input preparation, not part of the
    method's arithmetic.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def moe_layer(T, H, E, K, I, *, bf16: bool, seeds=(0, 1, 2, 3, 4),
              x_sigma=1.0, w_sigma=0.02):
    """One MoE layer's inputs: X [T,H], W_gu [E,2I,H], W_d [E,H,I], Wr [E,H],
    tgt [T,H].  ``seeds`` = (X, W_gu, W_d, Wr, tgt).  Wr stays fp32 (the router
    master copy is fp32 in every configuration); everything else is rounded to
    bf16 values when ``bf16``."""
    sx, sgu, sd, sr, st = seeds
    X = normal((T, H), x_sigma, sx)
    W_gu = normal((E, 2 * I, H), w_sigma, sgu)
    W_d = normal((E, H, I), w_sigma, sd)
    Wr = normal((E, H), w_sigma, sr)
    tgt = normal((T, H), 1.0, st)
    if bf16:
        X = to_bf16_values(X)
        W_gu = to_bf16_values(W_gu)
        W_d = to_bf16_values(W_d)
        tgt = to_bf16_values(tgt)
    return dict(X=X, W_gu=W_gu, W_d=W_d, Wr=Wr, tgt=tgt)


def flat_weights(W_gu: np.ndarray, W_d: np.ndarray) -> np.ndarray:
    """Concatenate the two fused expert tensors into one flat vector."""
    return np.concatenate([W_gu.ravel(), W_d.ravel()])


def random_mask(N: int, k: int, seed: int) -> np.ndarray:
    """``k`` distinct indices drawn uniformly from [0, N), sorted, uint32."""
    if k > N:
        raise ValueError("k > N")
    rng = _rng(seed)
    chosen = np.empty(0, dtype=np.int64)
    while chosen.size < k:
        need = k - chosen.size
        draw = rng.integers(0, N, size=need + need // 64 + 16, dtype=np.int64)
        chosen = np.unique(np.concatenate([chosen, draw]))
        if chosen.size > k:
            # drop a seeded random subset of the surplus so the result stays uniform
            drop = rng.choice(chosen.size, size=chosen.size - k, replace=False)
            chosen = np.delete(chosen, drop)
    return chosen.astype(np.uint32)


def quantize_affine_int4(W2d: np.ndarray, group: int = 128):
    """Min-max affine 4-bit quantiser used only to build the affine-dequant
    input: per group of ``group`` consecutive input-dim elements,
    scale = fp16((max - min) / 15) (1 for a constant group), zero =
    fp16(-min / scale), code = clip(rint(w / scale + zero), 0, 15); element 2i
    in the low nibble of byte i.  Returns (q_packed uint8 [rows, cols/2],
    scale_bits, zero_bits uint16 [rows, cols/group])."""
    rows, cols = W2d.shape
    if cols % group:
        raise ValueError("cols must be a multiple of the group size")
    g = W2d.reshape(rows, cols // group, group).astype(np.float32)
    lo, hi = g.min(axis=2), g.max(axis=2)
    span = (hi - lo) / np.float32(15.0)
    scale16 = np.where(span > 0, span, np.float32(1.0)).astype(np.float16)
    s = scale16.astype(np.float32)
    zero16 = (-lo / s).astype(np.float16)
    z = zero16.astype(np.float32)
    q = np.clip(np.rint(g / s[..., None] + z[..., None]), 0, 15).astype(np.uint8).reshape(rows, cols)
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale16.view(np.uint16), zero16.view(np.uint16)


def quantize_int4_g64(W2d: np.ndarray, group: int = 64):
    """Symmetric int4 quantiser used only to build the resident-dequant input.

    W2d: fp32 [rows, cols], cols % group == 0.
    Returns (q_packed uint8 [rows, cols/2], scale_bits uint16 [rows, cols/group])
    with scale = fp16(amax/7) per group and codes clamp(rint(w/scale), -7, 7);
    element 2i sits in the low nibble of byte i (two's complement).
    """
    rows, cols = W2d.shape
    if cols % group:
        raise ValueError("cols must be a multiple of the group size")
    g = W2d.reshape(rows, cols // group, group).astype(np.float32)
    amax = np.abs(g).max(axis=2)
    scale16 = (amax / np.float32(7.0)).astype(np.float16)
    s = scale16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1)), 0)
    q = np.clip(q, -7, 7).astype(np.int8).reshape(rows, cols)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale16.view(np.uint16)

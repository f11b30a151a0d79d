"""The routed-expert MXFP4 MoE layer, computed from its definition in fp64.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

For every token t and slot s (ascending), with e = topk_ids[t, s]:
  * e outside [0, E): the route is skipped, its weight ignored (exact zero;
    b12x PR #339, commit "FC2-only route validation").
  * otherwise, with W13_e = [w1_e; w3_e] (gate rows first, then up rows:
    "packed [gate; up] regions", pegainfer PR #867 commit 88ec37ec;
    "gate|up split-half", commit 53edfa98; "w1||w3", batchgen PR #307):
        g = w1_e x_t,  u = w3_e x_t,  h = silu(g) * u,  y = W2_e h,
        acc_t += w[t, s] * y
    with silu(z) = z / (1 + exp(-z)).
  * the weighted sum runs over slots in ascending order ("topk-slot-order
    accumulation", pegainfer PR #867, commit 53edfa98); tokens with no valid
    route get acc = +0.
Everything is fp64 with no intermediate rounding; x enters as its exact
bfloat16 value and the weights as their exact MXFP4 values.

MXFP8 variant: x (before FC1) and h (before FC2) are replaced by their MXFP8
round trip, blocks of 32 along K (``mxfp8_quantize``).

The whole-layer results are reached exactly by the definition; the per-expert
grouping below is only a way to evaluate it: each route's y is computed from
the same fp64 products and the slot-order sum is taken afterwards.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence, Tuple, Union

import numpy as np

from .formats import (bf16_bits_to_f64, dequant_mxfp4, e4m3_encode, e4m3_value,
                      e8m0_value, E4M3_MAX)

ExpertSource = Union[Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray],
                     Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]]]

MXFP8_BLOCK = 32


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------- MXFP8
def mxfp8_scale_exponent(amax: float) -> int:
    """Block scale exponent e = floor(log2(amax / 448)), found exactly by comparing
    amax with 448 * 2^e; clamped to [-127, 127]; amax == 0 gives -127.

    This is the literal scale rule of the MXFP8 x MXFP4 workload.  It puts the
    scaled block maximum in [448, 896), so the block maximum saturates to 448.
    """
    a = float(amax)
    if not np.isfinite(a):
        raise ValueError("non-finite block maximum")
    if a == 0.0:
        return -127
    _, ex = np.frexp(a)
    e = int(ex) - 1 - 9                 # 448 = 1.75 * 2^8, so e is near floor(log2 a) - 9
    while np.ldexp(E4M3_MAX, e + 1) <= a:
        e += 1
    while np.ldexp(E4M3_MAX, e) > a:
        e -= 1
    return max(-127, min(127, e))


def mxfp8_quantize(v: np.ndarray):
    """[..., K] fp64 -> (E4M3 codes uint8 [..., K], E8M0 bytes uint8 [..., K/32]).

    Per block of 32 along the last axis: e from ``mxfp8_scale_exponent``,
    codes = E4M3_RNE(saturate(v * 2^-e)), scale byte = e + 127 (pegainfer PR
    #867, commit 33d22f80: "gran-32 e4m3 activation quant" with UE8M0 scales).
    """
    x = np.asarray(v, dtype=np.float64)
    k = x.shape[-1]
    if k % MXFP8_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = x.reshape(-1, k // MXFP8_BLOCK, MXFP8_BLOCK)
    amax = np.abs(blocks).max(axis=2)
    exps = np.vectorize(mxfp8_scale_exponent, otypes=[np.int64])(amax) if amax.size else \
        np.zeros(amax.shape, np.int64)
    scaled = np.ldexp(blocks, -exps[:, :, None])
    codes = e4m3_encode(scaled).reshape(x.shape)
    scales = (exps + 127).astype(np.uint8).reshape(x.shape[:-1] + (k // MXFP8_BLOCK,))
    return codes, scales


def mxfp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = e4m3_value(codes)
    k = c.shape[-1]
    s = e8m0_value(scales)
    return (c.reshape(-1, k // MXFP8_BLOCK, MXFP8_BLOCK) * s.reshape(-1, k // MXFP8_BLOCK, 1)).reshape(c.shape)


def mxfp8_roundtrip(v: np.ndarray) -> np.ndarray:
    return mxfp8_dequantize(*mxfp8_quantize(v))


# --------------------------------------------------------------------------- forward
def _expert_getter(weights: ExpertSource):
    if callable(weights):
        return weights
    w13c, w13s, w2c, w2s = weights
    return lambda e: (w13c[e], w13s[e], w2c[e], w2s[e])


def expert_mlp(x_rows: np.ndarray, w13c, w13s, w2c, w2s, act: str = "bf16") -> np.ndarray:
    """y rows for one expert: W2 (silu(w1 x) * (w3 x)), fp64 throughout."""
    w13 = dequant_mxfp4(w13c, w13s)                  # [2I, H]
    inter = w13.shape[0] // 2
    gu = x_rows @ w13.T                               # [r, 2I]
    h = silu(gu[:, :inter]) * gu[:, inter:]
    if act == "mxfp8":
        h = mxfp8_roundtrip(h)
    w2 = dequant_mxfp4(w2c, w2s)                      # [H, I]
    return h @ w2.T                                   # [r, H]


def forward(hidden_bits: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
            weights: ExpertSource, experts: int, act: str = "bf16",
            tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp64 accumulator [len(tokens) or T, H] of the MoE layer.

    ``weights``: stacked checkpoint-layout arrays (w13_codes [E,2I,H/2],
    w13_scales [E,2I,H/32], w2_codes [E,H,I/2], w2_scales [E,H,I/32]) or a
    callable returning one expert's four arrays.  ``tokens``: evaluate only
    these tokens (rows of the result follow this order).
    """
    if act not in ("bf16", "mxfp8"):
        raise ValueError(f"unknown activation format {act!r}")
    get = _expert_getter(weights)
    ids = np.asarray(topk_ids, dtype=np.int64)
    wts = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    t_all, k = ids.shape
    sel = list(range(t_all)) if tokens is None else [int(t) for t in tokens]
    hidden = hidden_bits.shape[1]
    x = bf16_bits_to_f64(hidden_bits[sel]) if sel else np.zeros((0, hidden))
    if act == "mxfp8" and len(sel):
        x = mxfp8_roundtrip(x)

    # routes of the selected tokens, grouped by expert (ascending)
    by_expert = {}
    for i, t in enumerate(sel):
        for s in range(k):
            e = int(ids[t, s])
            if 0 <= e < experts:
                by_expert.setdefault(e, []).append((i, s))
    y = {}
    for e in sorted(by_expert):
        rows = by_expert[e]
        ye = expert_mlp(x[[i for i, _ in rows]], *get(e), act=act)
        for j, key in enumerate(rows):
            y[key] = ye[j]

    acc = np.zeros((len(sel), hidden), dtype=np.float64)
    for i, t in enumerate(sel):
        for s in range(k):                            # ascending slot order
            if (i, s) in y:
                acc[i] += wts[t, s] * y[(i, s)]
    return acc

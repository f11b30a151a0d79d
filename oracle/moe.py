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
round trip, blocks of 32 along K (``mxfp8_quantize``).  x is exact, so its
codes are unique; h is not: an implementation that holds h in fp32 may land
on the other side of a rounding decision where the exact h sits within fp32
rounding of one.  ``mxfp8_requant_check`` decides whether a given
quantisation of h is one of the correct ones, and ``forward(...,
h_requant=...)`` evaluates the rest of the layer from it.

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


def _roundtrip_at(blocks: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """MXFP8 round trip of [n, nb, 32] values with the given block exponents."""
    return np.ldexp(e4m3_value(e4m3_encode(np.ldexp(blocks, -exps[:, :, None]))), exps[:, :, None])


def mxfp8_requant_check(v: np.ndarray, dv: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> dict:
    """Whether (codes, scales) is an MXFP8 quantisation of some v' with
    |v' - v| <= dv elementwise, element by element.

    The quantiser is a step function of its input, so a value known only to
    within dv has more than one correct quantisation where the interval
    [v - dv, v + dv] straddles a decision: an E4M3 rounding midpoint of an
    element, or a scale boundary 448 * 2^e of its block maximum.  The block
    exponents any v' can give lie in [e_lo, e_hi] (those of the smallest and
    largest block maximum in the interval; the exponent rule is monotone), and
    at a given exponent the element's code lies between the codes of v - dv
    and v + dv (saturation and round-to-nearest-even are monotone).  An
    element is admissible when its block's scale byte is a reachable exponent
    and its value lies between those two codes' values at that exponent.

    Returns a dict: ``values`` (the dequantised (codes, scales)), ``rt`` (the
    round trip of v itself), ``admissible`` and ``ambiguous`` (bool arrays:
    more than one correct value exists for the element), and the counts
    ``n``, ``n_ambiguous``, ``n_differ`` (admissible values other than rt) and
    ``n_bad`` (inadmissible elements).
    """
    x = np.asarray(v, dtype=np.float64)
    d = np.broadcast_to(np.abs(np.asarray(dv, dtype=np.float64)), x.shape)
    k = x.shape[-1]
    if k % MXFP8_BLOCK:
        raise ValueError("K must be a multiple of 32")
    nb = k // MXFP8_BLOCK
    blocks = x.reshape(-1, nb, MXFP8_BLOCK)
    dblk = d.reshape(-1, nb, MXFP8_BLOCK)
    n = blocks.shape[0]
    expo = np.vectorize(mxfp8_scale_exponent, otypes=[np.int64])
    if blocks.size == 0:
        z = np.zeros(x.shape, bool)
        return dict(values=x.copy(), rt=x.copy(), admissible=~z, ambiguous=z, n=0, n_ambiguous=0,
                    n_differ=0, n_bad=0)
    mag = np.abs(blocks)
    e0 = expo(mag.max(axis=2))
    e_lo = expo(np.maximum(mag - dblk, 0.0).max(axis=2))
    e_hi = expo((mag + dblk).max(axis=2))
    rt = _roundtrip_at(blocks, e0)
    dev_e = np.asarray(scales, dtype=np.int64).reshape(n, nb) - 127
    got = mxfp8_dequantize(np.asarray(codes, dtype=np.uint8).reshape(n, nb * MXFP8_BLOCK),
                           np.asarray(scales, dtype=np.uint8).reshape(n, nb)).reshape(n, nb, MXFP8_BLOCK)
    lo = _roundtrip_at(blocks - dblk, dev_e)
    hi = _roundtrip_at(blocks + dblk, dev_e)
    reachable = ((dev_e >= e_lo) & (dev_e <= e_hi))[:, :, None]
    with np.errstate(invalid="ignore"):
        admissible = reachable & (got >= lo) & (got <= hi)
    # more than one correct value: several reachable exponents, or two codes at the exponent of v
    amb = (e_lo != e_hi)[:, :, None] | (_roundtrip_at(blocks - dblk, e0) != _roundtrip_at(blocks + dblk, e0))
    differ = admissible & (got != rt)
    shape = x.shape
    return dict(values=got.reshape(shape), rt=rt.reshape(shape), admissible=admissible.reshape(shape),
                ambiguous=amb.reshape(shape), n=int(x.size), n_ambiguous=int(amb.sum()),
                n_differ=int(differ.sum()), n_bad=int((~admissible).sum()))


def mxfp8_quantum(v: np.ndarray) -> np.ndarray:
    """Per element, the spacing of the E4M3 grid at v under v's own block
    exponent e (``mxfp8_quantize``): 2^(floor(log2 |v 2^-e|) - 3 + e) in the
    normal range (|v 2^-e| saturated to 448), 2^(-9 + e) below 2^-6."""
    x = np.asarray(v, dtype=np.float64)
    k = x.shape[-1]
    blocks = x.reshape(-1, k // MXFP8_BLOCK, MXFP8_BLOCK)
    if blocks.size == 0:
        return np.zeros_like(x)
    e = np.vectorize(mxfp8_scale_exponent, otypes=[np.int64])(np.abs(blocks).max(axis=2))[:, :, None]
    a = np.minimum(np.abs(np.ldexp(blocks, -e)), E4M3_MAX)
    _, ex = np.frexp(a)
    qe = np.where(a < 2.0 ** -6, -9, ex - 1 - 3)
    return np.ldexp(1.0, qe + e).reshape(x.shape)


# fp32 rounding of the h that the MXFP8 path requantises.  A K-long dot product
# evaluated as MFMA steps of at most 128 exact products (an adder tree of depth
# at most 7 with fp32 rounding) chained through an fp32 accumulator, with a few
# more fp32 additions for K split over waves, differs from the exact sum by at
# most (7 + ceil(K/128) + 4) * 2^-24 * sum|terms|; twice that is the allowance
# (it also covers truncating instead of rounding additions).  silu and the gate
# product add a few roundings of h on top (see ``h_uncertainty``).
FP32_EPS = 2.0 ** -24


def fp32_dot_bound(k: int) -> float:
    return 2.0 * (7 + -(-k // 128) + 4) * FP32_EPS


def _sigmoid(z):
    """1 / (1 + e^-z) without overflow and with full relative accuracy in both tails."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        ez = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + ez), ez / (1.0 + ez))


def silu_prime(z):
    """d/dz [z sigma(z)] = sigma(z) (1 + z sigma(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return _sigmoid(z) * (1.0 + z * _sigmoid(-z))


# silu'' = sigma' (2 + z (1 - 2 sigma)) vanishes at z = +-2.39935728...: the
# positive root of 2 + z tanh(-z / 2) = 0 (Newton from 2.4 to fp64 precision).
def _silu_prime_crit() -> float:
    z = 2.4
    for _ in range(60):
        f = 2.0 - z * np.tanh(0.5 * z)
        df = -np.tanh(0.5 * z) - 0.5 * z / np.cosh(0.5 * z) ** 2
        z -= f / df
    return float(z)


SILU_PRIME_CRIT = _silu_prime_crit()


def h_uncertainty(x_rows: np.ndarray, w13: np.ndarray, g: np.ndarray, u: np.ndarray, h: np.ndarray) -> np.ndarray:
    """Bound on |h_fp32 - h| for an fp32 evaluation of h = silu(g) * u whose
    g and u are fp32 dot products (``fp32_dot_bound``: |dg|, |du| <= gamma *
    sum|terms|) and whose silu runs on the hardware exponential.

    * g enters through silu: |silu(g') - silu(g)| <= dg * max|silu'| over
      [g - dg, g + dg] (mean value theorem).  |silu'| is monotone between the
      critical points of silu' (z = -c and z = c, c = 2.3994...), so its
      maximum on the interval is at an end or at a critical point inside.
      (The global bound |silu'| <= 1.1 would be far too loose where g << 0,
      where silu(g) ~ g e^g is tiny and flat.)
    * |silu(g') u' - silu(g) u| <= that * (|u| + du) + |silu(g)| du.
    * fp32 silu(z) = z * rcp(1 + exp(-z)) with exp(-z) = 2^(-z log2 e): the
      rounding of the exponent argument makes the exponential's relative error
      up to about 1.5 |z| ulp, plus the unit's own, the addition, the
      reciprocal and two products: (2 |z| + 10) ulp of h, taken generously.
    * g < -80: exp(-g) overflows fp32 and silu comes out as -0, so h is
      known only up to its own size there.
    """
    inter = g.shape[1]
    gam = fp32_dot_bound(x_rows.shape[1])
    absum = np.abs(x_rows) @ np.abs(w13).T            # sum of |terms| of every dot product
    dg, du = gam * absum[:, :inter], gam * absum[:, inter:]
    lo, hi = g - dg, g + dg
    dsilu = np.maximum(np.abs(silu_prime(lo)), np.abs(silu_prime(hi)))
    for c in (-SILU_PRIME_CRIT, SILU_PRIME_CRIT):
        dsilu = np.where((lo <= c) & (c <= hi), np.maximum(dsilu, abs(silu_prime(np.float64(c)))), dsilu)
    dh = dsilu * dg * (np.abs(u) + du) + np.abs(silu(g)) * du + (2.0 * np.abs(g) + 10.0) * FP32_EPS * np.abs(h)
    return np.where(g < -80.0, dh + np.abs(h), dh)


# --------------------------------------------------------------------------- forward
def _expert_getter(weights: ExpertSource):
    if callable(weights):
        return weights
    w13c, w13s, w2c, w2s = weights
    return lambda e: (w13c[e], w13s[e], w2c[e], w2s[e])


def expert_mlp(x_rows: np.ndarray, w13c, w13s, w2c, w2s, act: str = "bf16", h_requant=None):
    """y rows for one expert: W2 (silu(w1 x) * (w3 x)), fp64 throughout.

    MXFP8: h goes through its MXFP8 round trip before W2.  ``h_requant``
    (optional) replaces that round trip: it is called as ``h_requant(h, dh)``
    with the exact h rows and ``h_uncertainty`` of an fp32 evaluation, and
    returns the round-trip values to use (a checker passes the quantisation an
    implementation made, after ``mxfp8_requant_check`` has found it correct).
    """
    w13 = dequant_mxfp4(w13c, w13s)                  # [2I, H]
    inter = w13.shape[0] // 2
    gu = x_rows @ w13.T                               # [r, 2I]
    g, u = gu[:, :inter], gu[:, inter:]
    h = silu(g) * u
    w2 = dequant_mxfp4(w2c, w2s)                      # [H, I]
    if act == "mxfp8":
        if h_requant is None:
            h = mxfp8_roundtrip(h)
        else:
            h = h_requant(h, h_uncertainty(x_rows, w13, g, u, h))
    return h @ w2.T                                   # [r, H]


def forward(hidden_bits: np.ndarray, topk_ids: np.ndarray, topk_weights: np.ndarray,
            weights: ExpertSource, experts: int, act: str = "bf16",
            tokens: Optional[Sequence[int]] = None, h_requant=None, pool=None):
    """fp64 accumulator [len(tokens) or T, H] of the MoE layer.

    ``weights``: stacked checkpoint-layout arrays (w13_codes [E,2I,H/2],
    w13_scales [E,2I,H/32], w2_codes [E,H,I/2], w2_scales [E,H,I/32]) or a
    callable returning one expert's four arrays.  ``tokens``: evaluate only
    these tokens (rows of the result follow this order).  ``h_requant``
    (MXFP8 only): called as ``h_requant(e, routes, h, dh)`` per expert, with
    routes the (token, slot) pairs of h's rows; see ``expert_mlp``.  ``pool``:
    an executor whose ``map`` evaluates the experts' rows concurrently (each
    expert's rows are independent; the slot-order sum below is unchanged).
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
    order = sorted(by_expert)

    def one(e):
        rows = by_expert[e]
        hr = None
        if h_requant is not None:
            routes = [(sel[i], s) for i, s in rows]
            hr = lambda h, dh: h_requant(e, routes, h, dh)
        return expert_mlp(x[[i for i, _ in rows]], *get(e), act=act, h_requant=hr)

    results = list(pool.map(one, order)) if pool is not None else [one(e) for e in order]
    y = {}
    for e, ye in zip(order, results):
        for j, key in enumerate(by_expert[e]):
            y[key] = ye[j]

    acc = np.zeros((len(sel), hidden), dtype=np.float64)
    for i, t in enumerate(sel):
        for s in range(k):                            # ascending slot order
            if (i, s) in y:
                acc[i] += wts[t, s] * y[(i, s)]
    return acc

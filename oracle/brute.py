"""Scalar-loop brute force of the MoE layer for tiny shapes (pure Python).

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

Written separately from ``oracle.moe`` to pin it: E2M1 is decoded here by its
closed form (sign bit 3; magnitude m = code & 7 is 0.5*m when m < 2, else
2^((m >> 1) - 1) * (1 + (m & 1) / 2)) instead of the magnitude table, bf16
inputs by bit arithmetic in ``struct``, every dot product by an explicit loop
over k, and the route loop runs token by token in slot order with no grouping
by expert.  For the MXFP8 variant the activations are rounded by an
exhaustive nearest-value search over the E4M3 magnitudes.  Cost is
O(routes * 3 * I * H) Python operations: keep it to the tiny configuration.
"""
from __future__ import annotations

import math
import struct


def e2m1_closed_form(code: int) -> float:
    m = code & 7
    mag = 0.5 * m if m < 2 else 2.0 ** ((m >> 1) - 1) * (1.0 + (m & 1) / 2.0)
    return -mag if code & 8 else mag


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _weight(codes_row, scales_row, k: int) -> float:
    byte = int(codes_row[k // 2])
    code = (byte >> 4) if (k & 1) else (byte & 0xF)
    return e2m1_closed_form(code) * 2.0 ** (int(scales_row[k // 32]) - 127)


def _blocks_roundtrip(v):
    out = []
    for b in range(0, len(v), 32):
        out.extend(mxfp8_roundtrip_brute(v[b:b + 32])[0])
    return out


def forward_brute(hidden_bits, topk_ids, topk_weights, w13c, w13s, w2c, w2s, experts: int,
                  act: str = "bf16"):
    t_count, k_top = len(topk_ids), len(topk_ids[0]) if len(topk_ids) else 0
    hidden = len(hidden_bits[0]) if t_count else 0
    inter = len(w13c[0]) // 2 if len(w13c) else 0
    out = []
    for t in range(t_count):
        x = [_bf16(b) for b in hidden_bits[t]]
        if act == "mxfp8":
            x = _blocks_roundtrip(x)
        acc = [0.0] * hidden
        for s in range(k_top):
            e = int(topk_ids[t][s])
            if e < 0 or e >= experts:
                continue
            w = float(topk_weights[t][s])
            h = []
            for j in range(inter):
                g = sum(_weight(w13c[e][j], w13s[e][j], kk) * x[kk] for kk in range(hidden))
                u = sum(_weight(w13c[e][inter + j], w13s[e][inter + j], kk) * x[kk]
                        for kk in range(hidden))
                h.append(g / (1.0 + math.exp(-g)) * u)
            if act == "mxfp8":
                h = _blocks_roundtrip(h)
            for n in range(hidden):
                y = sum(_weight(w2c[e][n], w2s[e][n], kk) * h[kk] for kk in range(inter))
                acc[n] += w * y
        out.append(acc)
    return out


def _e4m3_finite_values():
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append((m * 2.0 ** -9) if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7))
    return vals  # ascending, 127 non-negative values, index = code


def mxfp8_roundtrip_brute(block):
    """MXFP8 round trip of one block by exhaustive search: the scale exponent is
    the largest e in [-127, 127] with 448 * 2^e <= amax (or -127), each element is
    saturated to 448 and then replaced by the nearest E4M3 magnitude, ties to the
    candidate with an even code."""
    vals = _e4m3_finite_values()
    amax = max(abs(float(v)) for v in block)
    e = -127
    if amax > 0:
        for cand in range(-127, 128):
            if 448.0 * 2.0 ** cand <= amax:
                e = cand
    out = []
    for v in block:
        a = min(abs(float(v)) * 2.0 ** (-e), 448.0)
        best = None
        for code, q in enumerate(vals):
            d = abs(a - q)
            if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
                best = (d, code, q)
        r = best[2] * 2.0 ** e
        out.append(-r if float(v) < 0 or (float(v) == 0 and math.copysign(1, float(v)) < 0) else r)
    return out, e + 127

"""Element and scale formats, written out from their definitions (fp64).

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

* E2M1 (MXFP4 element): 1 sign bit, 2 exponent bits, 1 mantissa bit; the eight
  magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (OCP Microscaling format
  specification, FP4 E2M1 element type).  Checkpoints store two elements per
  byte along K ("E2M1 nibbles + E8M0 scales", batchgen PR #307, section
  "What").  Nibble order: element 2j in bits 3:0, element 2j+1 in bits 7:4.
  The pages say the order was settled against an external library but do not
  print the verdict; the tests pin this order (and the whole dequantisation)
  bit for bit against an independently written MXFP4 decoder (transformers'
  MXFP4 integration), with the swapped order as a negative control.
* E8M0 (shared scale): an unsigned biased exponent, value 2^(b-127); the pages
  raise on the edge bytes 0x00 and 0xFF (batchgen PR #307, repack commit:
  "exact E8M0->bf16 expansion ... edge bytes raise"), so weight scales with
  those bytes are rejected by ``validate_scale_bytes``.
* E4M3FN (MXFP8 element): bias 7, no infinities, NaN = S.1111.111, largest
  finite 448, subnormal step 2^-9 (OCP 8-bit floating point specification).
* bfloat16: the upper 16 bits of an IEEE binary32.
"""
from __future__ import annotations

import numpy as np

E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E4M3_MAX = 448.0


# --------------------------------------------------------------------------- E2M1
def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] codes; element 2j from the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Inverse of ``unpack_nibbles``: [..., K] codes (0..15) -> [..., K/2] bytes."""
    c = np.asarray(codes, dtype=np.uint8)
    if c.shape[-1] % 2:
        raise ValueError("K must be even to pack E2M1 pairs")
    if np.any(c > 15):
        raise ValueError("E2M1 codes must be in 0..15")
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """Decode E2M1 codes (0..15) with the eight-value magnitude table; code 8 is -0."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = np.asarray(E2M1_MAGNITUDES, dtype=np.float64)[c & 7]
    return np.where(c & 8, -mag, mag)


# --------------------------------------------------------------------------- E8M0
def e8m0_value(b: np.ndarray) -> np.ndarray:
    """2^(b-127) in fp64 for b in 0..254; 0xFF is NaN."""
    bb = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, bb - 127)
    return np.where(bb == 255, np.nan, v)


def validate_scale_bytes(scales: np.ndarray, what: str = "scales") -> None:
    """Raise ValueError naming the first E8M0 byte equal to 0x00 or 0xFF."""
    s = np.asarray(scales, dtype=np.uint8)
    bad = (s == 0x00) | (s == 0xFF)
    if bad.any():
        idx = tuple(int(i) for i in np.argwhere(bad)[0])
        raise ValueError(f"{what}: E8M0 byte 0x{int(s[idx]):02X} at index {idx} is not accepted")


# --------------------------------------------------------------------------- MXFP4 tensor
def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Checkpoint-layout MXFP4 weights -> fp64 [N, K].

    codes [N, K/2] (row-major, K-major), scales [N, K/32]; one E8M0 scale per
    32 consecutive K elements of a row ("gran_k B=32", pegainfer PR #867,
    commit b49a9f04).  W[n, k] = E2M1(code[n, k]) * 2^(S[n, k // 32] - 127).
    """
    c = unpack_nibbles(codes)
    n, k = c.shape
    if k % 32 or scales.shape != (n, k // 32):
        raise ValueError(f"scales shape {scales.shape} does not match codes {codes.shape}")
    validate_scale_bytes(scales)
    w = e2m1_value(c).reshape(n, k // 32, 32)
    return (w * e8m0_value(scales)[:, :, None]).reshape(n, k)


# --------------------------------------------------------------------------- E4M3FN
def e4m3_value(codes: np.ndarray) -> np.ndarray:
    """Decode all E4M3FN codes to fp64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp64 -> E4M3FN codes: saturate |v| to 448, then round to nearest even
    (subnormals included).  The sign of a value that rounds to zero is kept."""
    x = np.asarray(v, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # quantum: 2^-9 below the smallest normal 2^-6, else 2^(floor(log2 a) - 3)
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e_floor = ex - 1
    quantum_exp = np.where(a < 2.0 ** -6, -9, e_floor - 3)
    q = np.rint(np.ldexp(a, -quantum_exp))     # exact scaling, then round-half-even
    val = np.ldexp(q, quantum_exp)             # the rounded magnitude (may reach the next binade)
    _, ex2 = np.frexp(val)
    e2 = ex2 - 1
    normal = val >= 2.0 ** -6
    sub_code = np.ldexp(val, 9)                # 0..8; 8 encodes 2^-6 as exponent 1, mantissa 0
    mant = np.where(normal, np.ldexp(val, -e2) * 8 - 8, 0)
    norm_code = ((e2 + 7) << 3) + mant.astype(np.int64)
    mag_code = np.where(normal, norm_code, sub_code.astype(np.int64))
    return (mag_code | np.where(sign, 0x80, 0)).astype(np.uint8)


# --------------------------------------------------------------------------- bfloat16
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns, round to nearest even; NaN stays NaN."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), rounded)


def ulp_bf16(ref: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at |ref|: 2^(max(floor(log2|ref|), -126) - 7)."""
    r = np.abs(np.asarray(ref, dtype=np.float64))
    _, ex = np.frexp(r)
    e = np.where(r > 0, ex - 1, -126)
    return np.ldexp(1.0, np.maximum(e, -126) - 7)

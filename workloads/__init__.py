"""Seeded synthetic inputs for the routed-expert MXFP4 MoE layer.

This module is shared by the CPU oracle tests, the GPU parity tests and the
benchmark.  It holds no arithmetic of the method itself: it only draws random
inputs (hidden states, routes, route weights, weight codes and scale bytes) and
describes the five workload configurations.  Random quantities the method
consumes are produced here and passed to both sides as plain arrays.

Input recipe (all draws from numpy's PCG64 through a SeedSequence of the
listed integers, so every array is reproducible on any host):

* hidden states: N(0, 1) in float32, rounded to nearest-even bfloat16 by
  torch's CPU cast; returned as uint16 bit patterns.
* routes: per token ``k`` expert ids.  ``uniform`` draws ``k`` distinct ids
  uniformly from ``[0, E_global)``; ``softmax_topk`` takes the top-``k`` of
  ``E_global`` N(0,1) logits; ``zipf`` draws ``k`` distinct ids by Gumbel-top-k
  over a popularity ``rank**-s`` whose ranks are mapped to ids by a seeded
  permutation.  Ids ``>= E_resident`` are not resident (they contribute an
  exact zero); ``invalid_frac`` of all routes are then replaced, half by -1
  and half by uniform ids in ``[E_resident, E_global)``.
* route weights: softmax, in float32, over the ``k`` selected N(0,1) logits
  of each token (for ``softmax_topk`` the logits are the router's own).
* weights: per expert a fresh generator seeded by (seed, expert, tensor).
  Code bytes are uniform over 0..255, so each E2M1 nibble is uniform over all
  16 codes; scale bytes are uniform integers in ``[scale_lo, scale_hi]``.
  Layout is the checkpoint's: codes ``[N, K/2]`` row-major (two K-consecutive
  elements per byte), scales ``[N, K/32]``.  W13 has N = 2*I rows (gate rows
  first, then up rows) and K = H; W2 has N = H and K = I.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "LayerShape",
    "Case",
    "CONFIGS",
    "DECODE_M",
    "config_case",
    "K3_SHAPE",
    "K3_DECODE_M",
    "k3_case",
    "make_case",
    "gen_hidden",
    "gen_routes",
    "gen_logits",
    "gen_expert",
    "gen_experts",
]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    tokens: int
    hidden: int
    inter: int
    experts: int          # resident experts E
    experts_global: int   # ids are drawn from [0, experts_global)
    top_k: int


@dataclasses.dataclass
class Case:
    """One seeded problem instance.  Expert weights are produced lazily per
    expert (``expert(e)``) so a sampled check never needs all of them."""

    name: str
    shape: LayerShape
    seed: int
    hidden_bits: np.ndarray        # uint16 [T, H], bfloat16 bit patterns
    topk_ids: np.ndarray           # int32 [T, k]
    topk_weights: np.ndarray       # float32 [T, k]
    scale_lo: int
    scale_hi: int
    act: str = "bf16"              # "bf16" or "mxfp8"
    nan_accumulator: bool = False  # caller's fp32 accumulator starts as NaN
    weight_seed: Optional[int] = None  # defaults to seed

    @property
    def wseed(self) -> int:
        return self.seed if self.weight_seed is None else self.weight_seed

    def expert(self, e: int):
        s = self.shape
        return gen_expert(self.wseed, e, s.hidden, s.inter, self.scale_lo, self.scale_hi)

    def experts(self):
        s = self.shape
        return gen_experts(self.wseed, s.experts, s.hidden, s.inter, self.scale_lo, self.scale_hi)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def gen_hidden(seed: int, tokens: int, hidden: int) -> np.ndarray:
    """bfloat16 bit patterns [tokens, hidden] of N(0,1) draws (RNE via torch)."""
    import torch

    x = _rng(seed, 1).standard_normal((tokens, hidden), dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _softmax_rows(logits: np.ndarray) -> np.ndarray:
    z = logits.astype(np.float32)
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z, dtype=np.float32)
    return (ez / ez.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)


def gen_routes(seed: int, tokens: int, top_k: int, experts: int, experts_global: int,
               kind: str = "uniform", zipf_s: float = 1.2, invalid_frac: float = 0.0):
    """Return (topk_ids int32 [T,k], topk_weights float32 [T,k])."""
    rng = _rng(seed, 2)
    if tokens == 0:
        return np.zeros((0, top_k), np.int32), np.zeros((0, top_k), np.float32)
    if kind == "softmax_topk":
        logits = rng.standard_normal((tokens, experts_global), dtype=np.float32)
        ids = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
        sel = np.take_along_axis(logits, ids, axis=1)
        w = _softmax_rows(sel)
    elif kind == "uniform":
        keys = rng.random((tokens, experts_global))
        ids = np.argsort(keys, axis=1, kind="stable")[:, :top_k]
        w = _softmax_rows(rng.standard_normal((tokens, top_k), dtype=np.float32))
    elif kind == "zipf":
        ranks = np.arange(1, experts + 1, dtype=np.float64)
        pop_by_rank = ranks ** (-zipf_s)
        perm = rng.permutation(experts)        # rank r -> expert id perm[r]
        logp = np.empty(experts)
        logp[perm] = np.log(pop_by_rank / pop_by_rank.sum())
        gumbel = -np.log(-np.log(rng.random((tokens, experts))))
        ids = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :top_k]
        w = _softmax_rows(rng.standard_normal((tokens, top_k), dtype=np.float32))
    else:
        raise ValueError(f"unknown routing kind {kind!r}")
    ids = ids.astype(np.int32)
    if invalid_frac > 0.0:
        n = ids.size
        nbad = int(round(invalid_frac * n))
        where = rng.choice(n, size=nbad, replace=False)
        flat = ids.reshape(-1)
        half = nbad // 2
        flat[where[:half]] = -1
        hi = max(experts_global, experts + 1)
        flat[where[half:]] = rng.integers(experts, hi, size=nbad - half, dtype=np.int32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w.astype(np.float32))


def gen_logits(seed: int, tokens: int, experts: int, ties: bool = False, specials: bool = False):
    """Router logits fp32 [T, E]: N(0,1); ``ties`` rounds them to multiples of
    1/4 (many exact ties); ``specials`` sets about 2% of them to NaN or -inf."""
    rng = _rng(seed, 5)
    lg = rng.standard_normal((tokens, experts), dtype=np.float32)
    if ties:
        lg = (np.round(lg * 4) / 4).astype(np.float32)
    if specials and lg.size:
        n = max(1, lg.size // 50)
        flat = lg.reshape(-1)
        where = rng.choice(lg.size, size=n, replace=False)
        flat[where[: n // 2]] = np.nan
        flat[where[n // 2:]] = -np.inf
    return np.ascontiguousarray(lg)


def gen_expert(seed: int, e: int, hidden: int, inter: int, scale_lo: int, scale_hi: int):
    """One expert's checkpoint-layout tensors:
    (w13_codes [2I, H/2], w13_scales [2I, H/32], w2_codes [H, I/2], w2_scales [H, I/32])."""
    r13 = _rng(seed, 3, e, 13)
    r2 = _rng(seed, 3, e, 2)
    w13c = np.frombuffer(r13.bytes(2 * inter * hidden // 2), dtype=np.uint8).reshape(2 * inter, hidden // 2)
    w13s = r13.integers(scale_lo, scale_hi + 1, size=(2 * inter, hidden // 32), dtype=np.uint8)
    w2c = np.frombuffer(r2.bytes(hidden * inter // 2), dtype=np.uint8).reshape(hidden, inter // 2)
    w2s = r2.integers(scale_lo, scale_hi + 1, size=(hidden, inter // 32), dtype=np.uint8)
    return w13c, w13s, w2c, w2s


def gen_experts(seed: int, experts: int, hidden: int, inter: int, scale_lo: int, scale_hi: int):
    """All experts stacked: ([E,2I,H/2], [E,2I,H/32], [E,H,I/2], [E,H,I/32])."""
    w13c = np.empty((experts, 2 * inter, hidden // 2), np.uint8)
    w13s = np.empty((experts, 2 * inter, hidden // 32), np.uint8)
    w2c = np.empty((experts, hidden, inter // 2), np.uint8)
    w2s = np.empty((experts, hidden, inter // 32), np.uint8)
    for e in range(experts):
        a, b, c, d = gen_expert(seed, e, hidden, inter, scale_lo, scale_hi)
        w13c[e], w13s[e], w2c[e], w2s[e] = a, b, c, d
    return w13c, w13s, w2c, w2s


def make_case(name: str, shape: LayerShape, seed: int, routing: str = "uniform",
              scale_lo: int = 120, scale_hi: int = 130, invalid_frac: float = 0.0,
              zipf_s: float = 1.2, act: str = "bf16", nan_accumulator: bool = False,
              weight_seed: Optional[int] = None) -> Case:
    x = gen_hidden(seed, shape.tokens, shape.hidden)
    ids, w = gen_routes(seed, shape.tokens, shape.top_k, shape.experts, shape.experts_global,
                        kind=routing, zipf_s=zipf_s, invalid_frac=invalid_frac)
    return Case(name, shape, seed, x, ids, w, scale_lo, scale_hi, act, nan_accumulator, weight_seed)


DECODE_M = (1, 4, 16, 64, 128)

# The five workload configurations (hidden 7168 / intermediate 2048 / top-8
# for 1-4; config 0 is the tiny case the oracle finishes in well under a second).
CONFIGS: Dict[int, dict] = {
    0: dict(name="tiny", shape=LayerShape(16, 256, 128, 8, 8, 2), routing="softmax_topk",
            scale_lo=120, scale_hi=130),
    1: dict(name="decode", shape=LayerShape(None, 7168, 2048, 224, 384, 8), routing="uniform",
            scale_lo=120, scale_hi=130),
    2: dict(name="prefill1536", shape=LayerShape(1536, 7168, 2048, 224, 224, 8), routing="uniform",
            scale_lo=118, scale_hi=132),
    3: dict(name="fusedsum4096", shape=LayerShape(4096, 7168, 2048, 224, 384, 8), routing="zipf",
            scale_lo=120, scale_hi=130, invalid_frac=0.01, nan_accumulator=True),
    4: dict(name="mxfp8x4096", shape=LayerShape(4096, 7168, 2048, 384, 384, 8), routing="uniform",
            scale_lo=120, scale_hi=130, act="mxfp8"),
}


def config_case(cid: int, m: Optional[int] = None, seed: Optional[int] = None) -> Case:
    """The seeded instance of configuration ``cid`` (decode needs ``m``).
    Default seed of activations and routes: 1000*cid + m for decode, 1000*cid
    otherwise; expert weights always use 1000*cid, so every decode batch size
    runs over the same experts."""
    c = dict(CONFIGS[cid])
    shape: LayerShape = c.pop("shape")
    name = c.pop("name")
    if cid == 1:
        if m is None:
            raise ValueError("decode configuration needs m")
        shape = dataclasses.replace(shape, tokens=int(m))
        name = f"{name}_m{m}"
    if seed is None:
        seed = 1000 * cid + (int(m) if cid == 1 else 0)
    return make_case(name, shape, seed, weight_seed=1000 * cid, **c)


# The pages' own expert shapes (Kimi K3, pegainfer PR #867, commit b49a9f04:
# W13 N=6144 / K=3584, W2 N=3584 / K=3072; top-16; 224 or 896 routed experts,
# batch buckets 1..128): one EP4 rank's share, 224 resident of 896, route ids
# uniform over all 896 (ids >= 224 contribute an exact zero).  Not one of the
# five configurations above; K3_PREFILL is a prefill-sized batch of the same
# shapes (bf16 or MXFP8 activations).
K3_SHAPE = LayerShape(None, 3584, 3072, 224, 896, 16)
K3_DECODE_M = (1, 16, 128)


def k3_case(m: int, act: str = "bf16") -> Case:
    shape = dataclasses.replace(K3_SHAPE, tokens=int(m))
    return make_case(f"k3_{act}_m{m}", shape, 6000 + int(m) + (500 if act == "mxfp8" else 0), routing="uniform",
                     act=act, weight_seed=6000)


def touched_experts(topk_ids: np.ndarray, experts: int) -> List[int]:
    """Distinct resident expert ids present in a routing (for byte accounting)."""
    v = topk_ids.reshape(-1)
    v = v[(v >= 0) & (v < experts)]
    return sorted(set(int(i) for i in np.unique(v)))

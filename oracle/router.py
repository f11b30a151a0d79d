"""Router top-k upstream of the layer: expert ids and route weights from router
logits.

TEST INFRASTRUCTURE ONLY: nothing in the product path may import this module.

The pages fix the contract, not the scoring function: a batched router top-k
over E in {224, 896} for batch buckets 1..128 (pegainfer PR #867, commit
b49a9f04), with the top-16 selection kept in registers, a fixed tie order and
the route weights' sequential FP32 normalisation (b12x PR #339, the paired
gather/router path).  Reading taken, the one the workloads' "top-k softmax"
routing uses:

  * ids: the k experts with the largest logits, in descending order; equal
    logits rank the lower expert id first; a NaN logit counts as -inf (in the
    ranking, ties again by id, and in the weights, where it gets 0);
  * weights: softmax over the k selected logits, max-subtracted:
        w_s = exp(l_s - l_0) / sum_{j=0..k-1} exp(l_j - l_0)
    with the sum taken over slots in ascending order.

Here both are computed in fp64 from the exact fp32 logits (``router_topk``);
the slot-by-slot scan with Python's ``sorted`` on the key (-logit, id) is the
definition written out, and the numpy formulation (``router_topk_np``) is a
second, independent one that pins it.
"""
from __future__ import annotations

import math

import numpy as np


def _rank_value(x: float) -> float:
    return -math.inf if math.isnan(x) else x


def router_topk(logits: np.ndarray, k: int):
    """(ids int32 [T, k], weights fp64 [T, k]) from fp32 logits [T, E]."""
    lg = np.asarray(logits, dtype=np.float32)
    t_all, e_all = lg.shape
    if not 1 <= k <= e_all:
        raise ValueError(f"k must be in [1, {e_all}], got {k}")
    ids = np.zeros((t_all, k), np.int32)
    w = np.zeros((t_all, k), np.float64)
    for t in range(t_all):
        row = [float(v) for v in lg[t]]
        order = sorted(range(e_all), key=lambda e: (-_rank_value(row[e]), e))[:k]
        ids[t] = order
        sel = [_rank_value(row[e]) for e in order]
        top = sel[0]
        ex = [math.exp(v - top) if not math.isnan(v - top) else math.nan for v in sel]
        total = 0.0
        for v in ex:                       # slots in ascending order
            total += v
        w[t] = [v / total for v in ex]
    return ids, w


def router_topk_np(logits: np.ndarray, k: int):
    """The same selection through numpy's stable argsort (NaN mapped to -inf)."""
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    lg = np.where(np.isnan(lg), -np.inf, lg)
    ids = np.argsort(-lg, axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = np.take_along_axis(lg, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ids, ex / ex.sum(axis=1, keepdims=True)

"""Helpers for the GPU parity tests: move seeded cases to the device, build
plans through the binding, and invert the repacked weight layout on the CPU.

The inverse below is written from the layout description of the library
(16-row x 128-K tiles, lane l owns row 16*nb + l%16 and checkpoint bytes
64*kb + 16*(l//16) .. +16; scales grouped by four column blocks, byte 4l+j =
group 4*(4c+j) + l//16; FC1 row blocks alternate gate j / up j).  It is test
code, independent of the kernels it checks.
"""
from __future__ import annotations

import numpy as np
import torch

import mxfp4_routed_expert_topk_amd as moe
import workloads as W
from workloads import device as D

ACT = {"bf16": moe.MOE_ACT_BF16, "mxfp8": moe.MOE_ACT_MXFP8}


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return D.to_dev(a, dev())


def upload_experts(case: W.Case):
    return D.upload_experts(case, dev())


def make_plan(case: W.Case, max_tokens=None, weights=None):
    s = case.shape
    cfg = moe.Config(s.hidden, s.inter, s.experts, s.top_k, max_tokens or max(1, s.tokens), ACT[case.act])
    w = weights if weights is not None else upload_experts(case)
    plan = moe.Plan(cfg, *w)
    return plan, w


def run_forward(plan, case: W.Case, with_acc=True, nan_acc=None, fused=False):
    x = to_dev(case.hidden_bits).view(torch.bfloat16)
    ids = to_dev(case.topk_ids)
    wts = to_dev(case.topk_weights)
    T, H = case.hidden_bits.shape
    acc = None
    if with_acc:
        fill = float("nan") if (case.nan_accumulator if nan_acc is None else nan_acc) else 0.0
        acc = torch.full((T, H), fill, dtype=torch.float32, device=dev())
    out = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device=dev())
    if fused:
        plan.forward_fused(x, ids, wts, out=out, acc=acc)
        plan.fused_status()   # synchronises; raises if a wait timed out
    else:
        plan.forward(x, ids, wts, out=out, acc=acc)
    torch.cuda.synchronize()
    return out, acc


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


# ----------------------------------------------------------------- repack inverse
def unrepack_codes(rp: np.ndarray, E: int, N: int, K: int, interleave_half: int = 0) -> np.ndarray:
    nb, kb = N // 16, K // 128
    t = rp[: E * nb * kb * 1024].reshape(E, nb, kb, 64, 16)
    out = np.zeros((E, N, K // 2), np.uint8)
    lane = np.arange(64)
    for b in range(nb):
        if interleave_half:
            rows = (interleave_half if b % 2 else 0) + (b // 2) * 16 + lane % 16
        else:
            rows = b * 16 + lane % 16
        for c in range(kb):
            cols = 64 * c + 16 * (lane // 16)
            for j in range(16):
                out[:, rows, cols + j] = t[:, b, c, :, j]
    return out


def unrepack_scales(rp: np.ndarray, E: int, N: int, K: int, interleave_half: int = 0):
    nb, kb = N // 16, K // 128
    kb4 = (kb + 3) // 4
    t = rp[: E * nb * kb4 * 256].reshape(E, nb, kb4, 64, 4)
    out = np.zeros((E, N, K // 32), np.uint8)
    pad_ok = True
    lane = np.arange(64)
    for b in range(nb):
        if interleave_half:
            rows = (interleave_half if b % 2 else 0) + (b // 2) * 16 + lane % 16
        else:
            rows = b * 16 + lane % 16
        for c in range(kb4):
            for j in range(4):
                k = 4 * c + j
                if k >= kb:
                    pad_ok &= bool((t[:, b, c, :, j] == 127).all())
                    continue
                out[:, rows, 4 * k + lane // 16] = t[:, b, c, :, j]
    return out, pad_ok

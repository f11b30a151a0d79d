"""Write tests/golden/tiny_forward.json: the oracle's fp64 output for the tiny
configuration (16 tokens, hidden 256, intermediate 128, 8 experts, top-2),
frozen with SHA-256 digests of its inputs and output so that a later change to
the oracle's arithmetic is seen.  Calls only ``oracle`` and ``workloads``.

The pages print no numeric example for this layer; the frozen digest plays the
part of the pinned oracle vector they describe (batchgen PR #307, repack
commit: a frozen verdict with sha256 pins), not an external truth.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def build():
    case = W.config_case(0)
    ew = case.experts()
    acc = oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights, ew, case.shape.experts)
    return {
        "config": "tiny: T=16 H=256 I=128 E=8 k=2, seed 0",
        "inputs_sha256": {
            "hidden_bits": digest(case.hidden_bits), "topk_ids": digest(case.topk_ids),
            "topk_weights": digest(case.topk_weights),
            "w13_codes": digest(ew[0]), "w13_scales": digest(ew[1]),
            "w2_codes": digest(ew[2]), "w2_scales": digest(ew[3]),
        },
        "acc_row0_first8_hex": [float(v).hex() for v in acc[0, :8]],
        "acc_row_l2": [float(np.linalg.norm(r)) for r in acc],
        "acc_f32_sha256": digest(acc.astype(np.float32)),
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_forward.json")
    with open(out, "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote", out)

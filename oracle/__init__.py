"""Plain fp64 CPU oracle of the routed-expert MXFP4 MoE layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
module and the benchmark's CPU-baseline leg may import anything here.  The
product path (the HIP library and its Python binding) never calls it, shares
no code with it and has no fallback to it.

Contents, each written from the definition on the pages (citations in each
module):
  formats  E2M1 / E8M0 / E4M3FN / bfloat16 codecs, MXFP4 dequantisation
  route    per-expert counts, offsets, stable permutation (two formulations)
  router   router top-k ids and softmax route weights from logits (upstream of the layer)
  moe      fp64 forward of the layer, MXFP8 activation quantisation
  brute    scalar-loop brute force for tiny shapes
  compare  the acceptance rule (3 bf16 ULP or 4e-3 row relative L2)

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
library codecs, brute force, exact invariants and, for the MXFP4
dequantisation including the nibble order inside a byte (element 2j in the low
nibble, which the pages settle without printing the verdict), an independently
written decoder (transformers' MXFP4 integration).
"""
from .formats import (E2M1_MAGNITUDES, E4M3_MAX, bf16_bits_to_f64, dequant_mxfp4, e2m1_value,
                      e4m3_encode, e4m3_value, e8m0_value, f32_to_bf16_rne, pack_nibbles,
                      ulp_bf16, unpack_nibbles, validate_scale_bytes)
from .route import route_sort, route_sort_by_key
from .router import router_topk, router_topk_np
from .moe import (expert_mlp, forward, fp32_dot_bound, mxfp8_dequantize, mxfp8_quantize, silu_prime,
                  mxfp8_requant_check, mxfp8_quantum, mxfp8_roundtrip, mxfp8_scale_exponent, silu, h_uncertainty)
from .compare import check_rows, rel_l2
from .brute import forward_brute, e2m1_closed_form

__all__ = [n for n in dir() if not n.startswith("_")]

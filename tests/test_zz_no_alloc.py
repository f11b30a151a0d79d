"""The allocation-free forward (moe_mxfp4_forward_noalloc) against the
workspace forward (moe_mxfp4_forward), through the C ABI: bitwise equal
outputs on two calls in a row, the second with fewer tokens (the fixed scratch
keeps the first call's contents), on the 16-row streaming kernels and on the
128-row-tile prefill kernels, and the capacity error for a batch whose scratch
would not fit."""
import numpy as np
import pytest
import torch

import mxfp4_routed_expert_topk_amd as moe
import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def _both(plan, case, T):
    x = G.to_dev(case.hidden_bits).view(torch.bfloat16)
    ids, wts = G.to_dev(case.topk_ids), G.to_dev(case.topk_weights)
    H = case.shape.hidden
    res = []
    for noalloc in (False, True):
        acc = torch.full((case.shape.tokens, H), float("nan"), dtype=torch.float32, device=x.device)
        out = torch.full((case.shape.tokens, H), float("nan"), dtype=torch.bfloat16, device=x.device)
        if noalloc:
            plan.forward_noalloc(x, ids, wts, out=out, acc=acc, num_tokens=T)
        else:
            plan.forward(x, ids, wts, out=out, acc=acc, num_tokens=T)
        torch.cuda.synchronize()
        res.append((G.bf16_bits(out)[:T], acc.cpu().numpy()[:T].view(np.uint32)))
    return res


@pytest.mark.parametrize("name,shape,seed,act,counts", [
    ("decode", W.LayerShape(64, 7168, 2048, 16, 24, 8), 81, "bf16", (64, 5)),
    ("prefill", W.LayerShape(300, 512, 384, 4, 4, 2), 82, "bf16", (300, 140)),
    ("decode_mx", W.LayerShape(40, 1024, 512, 8, 8, 4), 83, "mxfp8", (40, 9)),
    ("prefill_mx", W.LayerShape(300, 512, 384, 4, 6, 2), 84, "mxfp8", (300, 77)),
])
def test_noalloc_forward_matches_the_workspace_forward(name, shape, seed, act, counts):
    case = W.make_case(name, shape, seed, routing="uniform", invalid_frac=0.02, act=act)
    print(f"[gpu-test] noalloc {name} act={act} tokens {counts}", flush=True)
    plan, _ = G.make_plan(case)
    for T in counts:                  # the second call has fewer tokens
        (o_ws, a_ws), (o_na, a_na) = _both(plan, case, T)
        np.testing.assert_array_equal(o_na, o_ws)
        np.testing.assert_array_equal(a_na, a_ws)
        assert np.isfinite(a_na.view(np.float32)).all()


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    case = W.make_case("big", W.LayerShape(300, 7168, 2048, 2, 8, 8), 85)
    plan, _ = G.make_plan(case)
    x = G.to_dev(case.hidden_bits).view(torch.bfloat16)
    ids, wts = G.to_dev(case.topk_ids), G.to_dev(case.topk_weights)
    out = torch.empty((300, 7168), dtype=torch.bfloat16, device=x.device)
    with pytest.raises(moe.MoeError) as ei:
        plan.forward_noalloc(x, ids, wts, out=out)      # 300 tokens x top-8 at hidden 7168: ~79 MB of scratch
    assert ei.value.status == 4 and "bytes of scratch" in ei.value.message
    plan.forward_noalloc(x, ids, wts, out=out, num_tokens=0)   # an empty batch is a no-op

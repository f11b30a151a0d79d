"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every entry point include/moe_mxfp4.h declares, sizes buffers, and rejects
bad arguments with a status and a message before touching a device."""
import ctypes
import os
import re

import pytest
import torch

import mxfp4_routed_expert_topk_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mxfp4.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.fail(f"library not built at {moe.LIB_PATH}: run python -m mxfp4_routed_expert_topk_amd.build")
    return moe.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.moe_mxfp4_last_error() is not None


def cfg(**kw):
    base = dict(hidden=7168, intermediate=2048, num_experts=224, top_k=8, max_tokens=128, act=0)
    base.update(kw)
    return moe.Config(**base)


def test_query_sizes_decode_shape(lib):
    rp, ws = moe.query_sizes(cfg())
    # 224 experts x (codes + scales of W13 and W2); 23,396,352 bytes per expert
    # plus one 256-byte status word
    assert rp == 224 * 23_396_352 + 256
    assert ws >= 128 * 8 * 7168 * 4          # fp32 y rows
    rp2, _ = moe.query_sizes(cfg(hidden=256, intermediate=128, num_experts=8))
    # H=256 has 2 column blocks per row block, I=128 one: scale groups are padded
    # to 4 blocks (256 bytes per row block)
    per_expert = 16 * 2 * 1024 + 16 * 256 + 16 * 1 * 1024 + 16 * 256
    assert rp2 == 8 * per_expert + 256


@pytest.mark.parametrize("field,value,status,needle", [
    ("hidden", 7000, 2, "hidden must be a multiple of 128"),
    ("hidden", 0, 2, "hidden"),
    ("intermediate", 100, 2, "intermediate"),
    ("num_experts", 0, 2, "num_experts"),
    ("num_experts", 5000, 2, "num_experts"),
    ("top_k", 0, 2, "top_k"),
    ("top_k", 64, 2, "top_k"),
    ("max_tokens", 0, 2, "max_tokens"),
    ("act", 3, 1, "act must be"),
])
def test_config_validation(lib, field, value, status, needle):
    with pytest.raises(moe.MoeError) as ei:
        moe.query_sizes(cfg(**{field: value}))
    assert ei.value.status == status
    assert needle in ei.value.message
    assert str(value) in ei.value.message


def _plan_call(lib, c, ptrs, nbytes):
    h = ctypes.c_void_p()
    return lib.moe_mxfp4_plan(ctypes.byref(c.c()), *ptrs, nbytes, None, ctypes.byref(h)), h


def test_plan_argument_errors_before_any_device_call(lib):
    c = cfg(hidden=256, intermediate=128, num_experts=8, top_k=2, max_tokens=16)
    rp, _ = moe.query_sizes(c)
    st, _ = _plan_call(lib, c, [None, 16, 16, 16, 16], rp)
    assert st == 1 and b"w13_codes is null" in lib.moe_mxfp4_last_error()
    st, _ = _plan_call(lib, c, [16, 16, 16, 16, 24], rp)
    assert st == 3 and b"repacked must be 16-byte aligned" in lib.moe_mxfp4_last_error()
    st, _ = _plan_call(lib, c, [16, 16, 16, 16, 32], rp - 1)
    assert st == 6 and str(rp).encode() in lib.moe_mxfp4_last_error()


def test_forward_and_route_reject_null_plan(lib):
    assert lib.moe_mxfp4_forward(None, 16, 16, 16, 1, None, 16, 16, 1, None) == 1
    assert b"plan is null" in lib.moe_mxfp4_last_error()
    assert lib.moe_mxfp4_route(None, 16, 1, 16, 16, 16, 16, 16, 1, None) == 1
    assert lib.moe_mxfp4_set_stage_events(None, None, 0) == 1
    assert lib.moe_mxfp4_forward_fused(None, 16, 16, 16, 1, None, 16, 16, 1, None) == 1
    assert b"plan is null" in lib.moe_mxfp4_last_error()
    assert lib.moe_mxfp4_fused_status(None, 16, 1, None) == 1


def test_quantize_argument_errors(lib):
    assert lib.moe_mxfp8_quantize(16, 2, 33, 16, 16, None) == 2
    assert b"multiple of 32, got 33" in lib.moe_mxfp4_last_error()
    assert lib.moe_mxfp8_quantize(None, 2, 64, 16, 16, None) == 1
    assert lib.moe_mxfp8_quantize(16, 2, 64, 20, 16, None) == 3
    assert lib.moe_mxfp8_quantize(16, 0, 64, 16, 16, None) == 0     # empty is a no-op


def test_router_argument_errors(lib):
    assert lib.moe_router_topk(16, 4, 0, 1, 16, 16, None) == 2
    assert b"num_experts must be in [1, 1024], got 0" in lib.moe_mxfp4_last_error()
    assert lib.moe_router_topk(16, 4, 1025, 8, 16, 16, None) == 2
    assert lib.moe_router_topk(16, 4, 8, 9, 16, 16, None) == 2
    assert b"top_k must be in [1, min(32, num_experts=8)], got 9" in lib.moe_mxfp4_last_error()
    assert lib.moe_router_topk(16, 4, 896, 33, 16, 16, None) == 2
    assert lib.moe_router_topk(16, -1, 8, 2, 16, 16, None) == 1
    assert lib.moe_router_topk(None, 4, 8, 2, 16, 16, None) == 1
    assert lib.moe_router_topk(16, 4, 8, 2, 16, 24, None) == 3
    assert lib.moe_router_topk(16, 0, 8, 2, 16, 16, None) == 0       # no tokens: a no-op


def test_destroy_null_is_a_noop(lib):
    lib.moe_mxfp4_destroy(None)


def test_workspace_region_argument_errors(lib):
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.moe_mxfp4_workspace_region(None, 0, ctypes.byref(off), ctypes.byref(nb)) == 1
    assert b"plan is null" in lib.moe_mxfp4_last_error()


# ------------------------------------------------------------ binding argument checks (no device needed)
def _unbuilt_plan(**kw):
    """A Plan object with a configuration and a CPU workspace but no library
    plan behind it: enough for the binding's argument checks, which raise
    before any library call."""
    import torch
    p = object.__new__(moe.Plan)
    p.cfg = cfg(hidden=256, intermediate=128, num_experts=8, top_k=2, max_tokens=16, **kw)
    p.workspace = torch.zeros(1024, dtype=torch.uint8)
    p._h = ctypes.c_void_p()
    return p


def _good_args(T=4):
    import torch
    return dict(hidden=torch.zeros((T, 256), dtype=torch.bfloat16), topk_ids=torch.zeros((T, 2), dtype=torch.int32),
                topk_weights=torch.zeros((T, 2), dtype=torch.float32))


def _bad(**changes):
    import torch
    a = _good_args()
    a.update(changes)
    return a


@pytest.mark.parametrize("name,kw,needle", [
    ("int64 ids", lambda t: _bad(topk_ids=torch.zeros((4, 2), dtype=torch.int64)), "topk_ids must be torch.int32"),
    ("ids too few rows", lambda t: _bad(topk_ids=torch.zeros((3, 2), dtype=torch.int32)), "at least 4 rows"),
    ("ids wrong k", lambda t: _bad(topk_ids=torch.zeros((4, 3), dtype=torch.int32)), "2 columns"),
    ("fp16 weights", lambda t: _bad(topk_weights=torch.zeros((4, 2), dtype=torch.float16)), "topk_weights must be"),
    ("weights short", lambda t: _bad(topk_weights=torch.zeros((2, 2), dtype=torch.float32)), "at least 4 rows"),
    ("fp32 hidden", lambda t: _bad(hidden=torch.zeros((4, 256), dtype=torch.float32)), "hidden must be torch.bfloat16"),
    ("hidden width", lambda t: _bad(hidden=torch.zeros((4, 128), dtype=torch.bfloat16)), "256 columns"),
    ("strided hidden", lambda t: _bad(hidden=torch.zeros((4, 512), dtype=torch.bfloat16)[:, ::2]), "contiguous"),
    ("out short", lambda t: _bad(out=torch.zeros((2, 256), dtype=torch.bfloat16)), "out must have at least 4 rows"),
    ("acc dtype", lambda t: _bad(acc=torch.zeros((4, 256), dtype=torch.bfloat16)), "acc must be torch.float32"),
    ("acc short", lambda t: _bad(acc=torch.zeros((3, 256), dtype=torch.float32)), "acc must have at least 4 rows"),
    ("device", lambda t: _bad(topk_ids=torch.zeros((4, 2), dtype=torch.int32, device="meta")), "must be on cpu"),
    ("tokens past hidden", lambda t: dict(_good_args(), num_tokens=5), "num_tokens must be in [0, 4]"),
    ("negative tokens", lambda t: dict(_good_args(), num_tokens=-1), "num_tokens must be in [0, 4]"),
    ("workspace dtype", lambda t: dict(_good_args(), workspace=torch.zeros(64, dtype=torch.int32)), "workspace must be"),
])
def test_binding_rejects_bad_forward_arguments(lib, name, kw, needle):
    """int64 ids (torch.topk's default), short or mistyped tensors, strided
    views, another device, or a token count past the rows would make the
    kernels read or write out of bounds: the binding raises MOE_ERR_ARG first."""
    import torch
    p = _unbuilt_plan()
    for fn in (p.forward, p.forward_fused):
        with pytest.raises(moe.MoeError) as ei:
            fn(**kw(torch))
        assert ei.value.status == 1 and needle in ei.value.message, (name, ei.value.message)


def test_binding_rejects_bad_route_router_and_quantiser_arguments(lib):
    import torch
    p = _unbuilt_plan()
    with pytest.raises(moe.MoeError, match="topk_ids must be torch.int32"):
        p.route(torch.zeros((4, 2), dtype=torch.int64))
    with pytest.raises(moe.MoeError, match=r"num_tokens must be in \[0, 4\]"):
        p.route(torch.zeros((4, 2), dtype=torch.int32), num_tokens=9)
    with pytest.raises(moe.MoeError, match="logits must be torch.float32"):
        moe.router_topk(torch.zeros((4, 8), dtype=torch.float64), 2)
    with pytest.raises(moe.MoeError, match="topk_ids must have 2 columns"):
        moe.router_topk(torch.zeros((4, 8)), 2, ids=torch.zeros((4, 3), dtype=torch.int32))
    with pytest.raises(moe.MoeError, match="x must be torch.bfloat16"):
        moe.mxfp8_quantize(torch.zeros((4, 64)))

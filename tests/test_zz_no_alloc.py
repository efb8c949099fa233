"""moe_expert_forward_noalloc (static scratch, no allocation in the call)
against moe_expert_forward, called through the C ABI: bit-identical outputs on
two calls in a row, the second with a smaller batch, for the OLMoE-like and
the Qwen3-Next-like (shared expert) shapes; the second call is also checked
against the oracle.  A batch whose scratch exceeds the static array is refused
before anything is enqueued."""
import ctypes as C

import numpy as np
import pytest
import torch

from fixtures import moe_inputs as fx
from oracle import moe_oracle as ora

from gpu_util import assert_close, say

pytestmark = pytest.mark.gpu


def _p(t):
    return C.c_void_p(t.data_ptr())


def _calls(moe, ctx, x, ids, w):
    lib = moe.capi.load()
    T, H = x.shape
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = torch.full((T, H), float("nan"), dtype=torch.float16, device="cuda")
    got = torch.full((T, H), float("nan"), dtype=torch.float16, device="cuda")
    st = lib.moe_expert_forward(ctx._h, 0, _p(x), T, _p(ids), _p(w), _p(ref), s)
    assert st == moe.capi.MOE_OK, lib.moe_last_error(ctx._h)
    st = lib.moe_expert_forward_noalloc(ctx._h, 0, _p(x), T, _p(ids), _p(w), _p(got), s)
    assert st == moe.capi.MOE_OK, lib.moe_last_error(ctx._h)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("shape_name,sizes", [("OLMOE", (64, 7)), ("QWEN_NEXT", (16, 3))])
def test_noalloc_equals_expert_forward_two_calls(shape_name, sizes):
    import w4a16_routed_expert_router_amd as moe
    say(f"test_noalloc_equals_expert_forward_two_calls {shape_name} T={sizes}")
    shape = getattr(fx, shape_name)
    wts = {k: v.cpu().numpy() for k, v in
           fx.layer_weights(shape, "noalloc", 0, device="cuda", batched=True).items()}
    ctx = moe.MoEContext(shape, n_layers=1, max_tokens=max(sizes))
    ctx.register_layer(0, wts)
    for i, T in enumerate(sizes):
        x = fx.activations(("noalloc", shape_name, T), T, shape.hidden, device="cuda")
        ids, w = ctx.route(0, x)
        ref, got = _calls(moe, ctx, x, ids, w)
        assert torch.equal(ref, got), f"call {i} (T={T}) differs from moe_expert_forward"
        if i == 1:
            o = ora.moe_layer(x.cpu().numpy(), wts, shape)
            np.testing.assert_array_equal(ids.cpu().numpy(), o["ids"])
            assert_close(got.float().cpu().numpy(), o["out"], f"{shape_name} T={T} vs oracle")
    assert ctx.check_device_errors() == 0
    ctx.close()


def test_noalloc_refuses_batches_beyond_the_static_scratch():
    import w4a16_routed_expert_router_amd as moe
    say("test_noalloc_refuses_batches_beyond_the_static_scratch")
    shape = fx.MoEShape(hidden=2048, n_experts=64, inter=1024, top_k=8, renorm=False)
    wts = {k: v.cpu().numpy() for k, v in fx.layer_weights(shape, "noalloc-big", 0, device="cuda").items()}
    ctx = moe.MoEContext(shape, n_layers=1, max_tokens=128)
    ctx.register_layer(0, wts)
    lib = moe.capi.load()
    T = 100                                   # 99 tokens is the most this shape fits
    x = fx.activations(("noalloc-big",), T, shape.hidden, device="cuda")
    ids, w = ctx.route(0, x)
    out = torch.zeros((T, shape.hidden), dtype=torch.float16, device="cuda")
    torch.cuda.synchronize()
    st = lib.moe_expert_forward_noalloc(ctx._h, 0, _p(x), T, _p(ids), _p(w), _p(out),
                                        C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == moe.capi.MOE_E_ARG
    assert b"static scratch" in lib.moe_last_error(ctx._h)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0      # nothing was enqueued
    ctx.close()

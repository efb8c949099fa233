"""Residual MoE stacks on the GPU against the oracle.

Teacher-forced per layer: the GPU's own normalised input x_l of each layer is
routed by the oracle (ids must match bit for bit) and run through the oracle's
layer; the GPU's residual increment must match within the layer tolerance.
Free-running: final residuals of whole stacks within tolerance.
"""
import numpy as np
import pytest
import torch

from fixtures import moe_inputs as fx
from oracle import moe_oracle as ora

from gpu_util import assert_close, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import w4a16_routed_expert_router_amd as m
    return m


_CACHE = {}


def stack_weights(shape, cfg, L):
    key = (shape, cfg, L)
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = [{k: v.cpu().numpy() for k, v in
                        fx.layer_weights(shape, cfg, l, device="cuda", batched=True).items()}
                       for l in range(L)]
    return _CACHE[key]


def make_ctx(moe, shape, layers, T, flags=0, **kw):
    ctx = moe.MoEContext(shape, n_layers=len(layers), max_tokens=T, flags=flags, **kw)
    for l, w in enumerate(layers):
        ctx.register_layer(l, w)
    return ctx


def teacher_forced(ctx, shape, layers, h0, check_layers=None, forced=None):
    """Run layer by layer; check each layer against the oracle on the GPU's x."""
    T = h0.shape[0]
    h = torch.from_numpy(h0.astype(np.float32)).cuda()
    worst = 0.0
    fg = None if forced is None else torch.from_numpy(forced).cuda()
    for l in range(len(layers)):
        before = h.cpu().numpy().astype(np.float64)
        xs, ids, ws = ctx.stack_forward(h, l, l + 1, forced_ids=fg, trace=True)
        torch.cuda.synchronize()
        after = h.cpu().numpy().astype(np.float64)
        x = xs[l].cpu().numpy()
        # RMSNorm: the GPU's FP32 normalisation vs the oracle's FP64, both rounded to FP16
        xr = ora.rmsnorm_fp16(before)
        ulp = np.abs(x.astype(np.float32) - xr.astype(np.float32)) / np.spacing(np.abs(xr).astype(np.float16)).astype(np.float32)
        assert ulp.max() <= 1.0, (l, ulp.max())
        if check_layers is not None and l not in check_layers:
            continue
        ref = ora.moe_layer(x, layers[l], shape, None if forced is None else forced[l])
        np.testing.assert_array_equal(ids[l].cpu().numpy(), ref["ids"])
        np.testing.assert_allclose(ws[l].cpu().numpy(), ref["w"], rtol=1e-5, atol=1e-7)
        r, _ = assert_close(after - before, ref["out"], f"layer {l}")
        worst = max(worst, r)
    assert ctx.check_device_errors() == 0
    return h, worst


@pytest.mark.parametrize("fused", [True, False])
def test_olmoe_stack_decode_teacher_forced(moe, fused):
    """OLMoE-shaped 16-layer stack, batch 1, both execution paths."""
    say(f"test_olmoe_stack_decode_teacher_forced fused={fused}")
    shape, L = fx.OLMOE, 16
    layers = stack_weights(shape, "stack-olmoe", L)
    ctx = make_ctx(moe, shape, layers, 1, flags=0 if fused else moe.MOE_FLAG_NO_FUSED)
    for i in range(2):
        h0 = fx.activations(("stack-olmoe-h0", i), 1, shape.hidden).numpy()
        teacher_forced(ctx, shape, layers, h0, check_layers=range(L) if i == 0 else (0, 7, 15))
    ctx.close()


@pytest.mark.parametrize("T", [4, 8])
def test_olmoe_stack_batched_decode_fused(moe, T):
    say(f"test_olmoe_stack_batched_decode_fused T={T}")
    shape, L = fx.OLMOE, 16
    layers = stack_weights(shape, "stack-olmoe", L)
    ctx = make_ctx(moe, shape, layers, T)
    h0 = fx.activations(("stack-olmoe-T", T), T, shape.hidden).numpy()
    teacher_forced(ctx, shape, layers, h0, check_layers=(0, 5, 10, 15))
    ctx.close()


def test_olmoe_stack_whole_call_equals_layer_by_layer(moe):
    """One launch over all layers gives the same bits as one launch per layer."""
    say("test_olmoe_stack_whole_call_equals_layer_by_layer")
    shape, L = fx.OLMOE, 16
    layers = stack_weights(shape, "stack-olmoe", L)
    ctx = make_ctx(moe, shape, layers, 2)
    h0 = torch.from_numpy(fx.activations(("whole",), 2, shape.hidden).numpy().astype(np.float32)).cuda()
    a = h0.clone()
    ctx.stack_forward(a)
    b = h0.clone()
    for l in range(L):
        ctx.stack_forward(b, l, l + 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # and repeated calls are deterministic
    c = h0.clone()
    ctx.stack_forward(c)
    torch.cuda.synchronize()
    assert torch.equal(a, c)
    assert ctx.check_device_errors() == 0
    ctx.close()


@pytest.mark.parametrize("T", [1, 3])
def test_olmoe_stack_free_running_vs_oracle(moe, T):
    say(f"test_olmoe_stack_free_running_vs_oracle T={T}")
    shape, L = fx.OLMOE, 16
    layers = stack_weights(shape, "stack-olmoe", L)
    for fused in (True, False):
        ctx = make_ctx(moe, shape, layers, T, flags=0 if fused else moe.MOE_FLAG_NO_FUSED)
        h0 = fx.activations(("free", T), T, shape.hidden).numpy()
        h = torch.from_numpy(h0.astype(np.float32)).cuda()
        _, ids, _ = ctx.stack_forward(h, trace=True)
        torch.cuda.synchronize()
        ref = ora.stack_forward(h0, layers, shape)
        agree = np.mean([np.array_equal(ids[l].cpu().numpy(), ref["ids"][l]) for l in range(L)])
        say(f"  fused={fused}: layers with identical ids {agree:.3f}")
        if agree == 1.0:
            assert_close(h.cpu().numpy(), ref["h"], f"final h fused={fused}")
        else:   # a near-tie flipped by FP16 rounding upstream: report, teacher-forced tests decide
            say(f"  final h rel_l2 {rel_l2(h.cpu().numpy(), ref['h']):.3e} (routing diverged)")
        ctx.close()


@pytest.mark.parametrize("T", [1, 4])
def test_qwen_stack_decode_teacher_forced(moe, T):
    """Qwen3-Next-style layers (512 experts, top-10 renormalised, shared expert),
    8 of the 48 layers at full per-layer size."""
    say(f"test_qwen_stack_decode_teacher_forced T={T}")
    shape, L = fx.QWEN_NEXT, 8
    layers = stack_weights(shape, "stack-qwen", L)
    ctx = make_ctx(moe, shape, layers, T)
    h0 = fx.activations(("stack-qwen-h0", T), T, shape.hidden).numpy()
    teacher_forced(ctx, shape, layers, h0, check_layers=(0, 3, 7))
    ctx.close()


def test_qwen_stack_batch16_per_layer_kernels(moe):
    """Batch 16 takes the per-layer kernels (16 tokens x top-10 > 64 pairs)."""
    say("test_qwen_stack_batch16_per_layer_kernels")
    shape, L = fx.QWEN_NEXT, 8
    layers = stack_weights(shape, "stack-qwen", L)
    ctx = make_ctx(moe, shape, layers, 16)
    h0 = fx.activations(("stack-qwen-16",), 16, shape.hidden).numpy()
    teacher_forced(ctx, shape, layers, h0, check_layers=(0, 7))
    ctx.close()


def test_stack_forced_trace_both_paths(moe):
    """Trace-driven routing: ids are the trace; both paths match the oracle."""
    say("test_stack_forced_trace_both_paths")
    shape, L = fx.OLMOE, 16
    layers = stack_weights(shape, "stack-olmoe", L)
    trace = fx.zipf_trace("stack-forced", 1, L, shape.n_experts, shape.top_k)[0][:, None, :]
    h0 = fx.activations(("forced-h0",), 1, shape.hidden).numpy()
    for flags in (0, moe.MOE_FLAG_NO_FUSED):
        ctx = make_ctx(moe, shape, layers, 1, flags=flags)
        teacher_forced(ctx, shape, layers, h0, check_layers=(0, 8, 15), forced=np.ascontiguousarray(trace))
        ctx.close()

"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: routing indices and cache decisions bit-exact; router logits bit-exact
(both sides compute the FP32 value nearest to the exact dot product); combine
weights within 1e-5 relative; layer outputs within relative L2 2e-3 and
max-abs 5e-2 of the float64 oracle.
"""
import numpy as np
import pytest
import torch

from fixtures import moe_inputs as fx
from oracle import moe_oracle as ora

from gpu_util import assert_close, gpu_layer, say, to_gpu

pytestmark = pytest.mark.gpu

SMALL = fx.MoEShape(hidden=256, n_experts=16, inter=256, top_k=4, renorm=False)
SMALL_SHARED = fx.MoEShape(hidden=512, n_experts=32, inter=256, top_k=3, renorm=True, shared_inter=512)


@pytest.fixture(scope="module")
def moe():
    import w4a16_routed_expert_router_amd as m
    assert torch.cuda.is_available()
    return m


def _ctx(m, shape, n_layers=1, max_tokens=64, **kw):
    return m.MoEContext(shape, n_layers=n_layers, max_tokens=max_tokens, **kw)


def _check_route(ctx, wts, shape, x, forced=None):
    ids, w, lg = ctx.route(0, to_gpu(x), forced_ids=None if forced is None else to_gpu(forced),
                           want_logits=True)
    torch.cuda.synchronize()
    o_ids, o_w, o_lg = ora.route(x, wts["router"], shape.top_k, shape.renorm, forced)
    if forced is None:
        np.testing.assert_array_equal(lg.cpu().numpy().view(np.uint32), o_lg.view(np.uint32))
    np.testing.assert_array_equal(ids.cpu().numpy(), o_ids)
    np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=1e-5, atol=1e-7)
    return ids, w


@pytest.mark.parametrize("T", [1, 5, 37])
def test_route_small(moe, T):
    say(f"test_route_small T={T}")
    wts = gpu_layer(SMALL, "gpu-small", 0)
    ctx = _ctx(moe, SMALL)
    ctx.register_layer(0, wts)
    x = fx.activations(("route-small", T), T, SMALL.hidden).numpy()
    _check_route(ctx, wts, SMALL, x)
    assert ctx.check_device_errors() == 0


def test_route_ties_pick_lowest_id(moe):
    say("test_route_ties_pick_lowest_id")
    wts = gpu_layer(SMALL, "gpu-ties", 0)
    wts["router"][9] = wts["router"][2]
    wts["router"][12] = wts["router"][2]
    ctx = _ctx(moe, SMALL)
    ctx.register_layer(0, wts)
    x = np.sign(wts["router"][2:3].astype(np.float32)).astype(np.float16).repeat(3, 0)
    ids, _ = _check_route(ctx, wts, SMALL, x)
    assert ids.cpu().numpy()[0, :3].tolist() == [2, 9, 12]


@pytest.mark.parametrize("flags", [0, 1])
def test_route_olmoe_qwen_shapes(moe, flags):
    say(f"test_route_olmoe_qwen_shapes flags={flags}")
    for shape, T in ((fx.OLMOE, 64), (fx.OLMOE, 512), (fx.QWEN_NEXT, 16)):
        router = fx.router_only(shape, "gpu-route", 0, device="cuda").cpu().numpy()
        wts = {"router": router}
        ctx = moe.MoEContext(shape, n_layers=1, max_tokens=T, flags=flags)
        # router-only registration: zero experts (never run here)
        E, H, I = shape.n_experts, shape.hidden, shape.inter
        full = {"router": router, "q": np.zeros((E, 3, I * H // 2), np.uint8),
                "s": np.zeros((E, 3, I * H // 128), np.float16)}
        if shape.shared_inter:
            full["shared_q"] = np.zeros((3, shape.shared_inter * H // 2), np.uint8)
            full["shared_s"] = np.zeros((3, shape.shared_inter * H // 128), np.float16)
        ctx.register_layer(0, full)
        x = fx.activations(("route-shapes", T), T, H).numpy()
        ids, w = _check_route(ctx, wts, shape, x)
        if shape.renorm:
            np.testing.assert_allclose(w.sum(1).cpu().numpy(), 1.0, rtol=1e-5)
        ctx.close()


def test_route_wide_range_inputs_exact(moe):
    """Inputs spanning FP16 subnormals to large values stress the exact tier."""
    say("test_route_wide_range_inputs_exact")
    rng = np.random.default_rng(3)
    wts = gpu_layer(SMALL, "gpu-wide", 0)
    bits = rng.integers(0, 1 << 16, size=(8, SMALL.hidden), dtype=np.uint16)
    x = bits.view(np.float16)
    x = np.where(np.isfinite(x), x, np.float16(0.5)).astype(np.float16)
    x = np.clip(x, -2.0, 2.0).astype(np.float16)   # keep logits finite
    wts["router"] = np.where(np.arange(SMALL.hidden) % 3 == 0, wts["router"] * np.float16(1e-3),
                             wts["router"]).astype(np.float16)
    ctx = _ctx(moe, SMALL)
    ctx.register_layer(0, wts)
    _check_route(ctx, wts, SMALL, x)


def test_route_midpoint_logits_round_to_even(moe):
    """Exact sums on an FP32 rounding midpoint: no FP64 error interval can be
    certified there, so these logits take the exact tier and must round to even."""
    say("test_route_midpoint_logits_round_to_even")
    wts = gpu_layer(SMALL, "gpu-mid", 0)
    H = SMALL.hidden
    router = np.zeros((SMALL.n_experts, H), np.float16)
    router[:, 0] = 1.0
    router[:, 1] = np.float16(2.0 ** -24)              # smallest FP16 subnormal
    router[:, 2] = np.arange(SMALL.n_experts) % 4      # 0..3 ulps of 1.0 at 2^-23
    wts["router"] = router
    x = np.zeros((3, H), np.float16)
    x[:, 0] = 1.0
    x[:, 1] = 1.0                                      # + 2^-24: half an ulp of 1.0
    x[:, 2] = np.float16(2.0 ** -23)
    x[1, 0] = 2.0                                      # 2 + 2^-24: a quarter ulp, not a midpoint
    x[2, 3] = 1.0                                      # unused column
    ctx = _ctx(moe, SMALL)
    ctx.register_layer(0, wts)
    _check_route(ctx, wts, SMALL, x)
    _, _, lg = ctx.route(0, to_gpu(x), want_logits=True)
    lg = lg.cpu().numpy()
    # token 0, expert 0: 1 + 2^-24 rounds to even (1.0); expert 1: 1 + 2^-23 + 2^-24 rounds up
    assert lg[0, 0] == np.float32(1.0)
    assert lg[0, 1] == np.float32(1.0 + 2.0 ** -22)


def test_route_forced_ids_gather_softmax(moe):
    say("test_route_forced_ids_gather_softmax")
    wts = gpu_layer(SMALL, "gpu-forced", 0)
    ctx = _ctx(moe, SMALL)
    ctx.register_layer(0, wts)
    T = 9
    x = fx.activations(("forced",), T, SMALL.hidden).numpy()
    rng = np.random.default_rng(0)
    forced = np.stack([np.sort(rng.choice(SMALL.n_experts, SMALL.top_k, replace=False))
                       for _ in range(T)]).astype(np.int32)
    _check_route(ctx, wts, SMALL, x, forced)
    assert ctx.check_device_errors() == 0


def test_route_forced_bad_ids_set_error_word(moe):
    say("test_route_forced_bad_ids_set_error_word")
    wts = gpu_layer(SMALL, "gpu-forced", 0)
    ctx = _ctx(moe, SMALL)
    ctx.register_layer(0, wts)
    x = fx.activations(("forced-bad",), 2, SMALL.hidden).cuda()
    forced = torch.tensor([[0, 1, 2, 99], [3, 3, 4, 5]], dtype=torch.int32, device="cuda")
    ids, _ = ctx.route(0, x, forced_ids=forced)
    bits = ctx.check_device_errors()
    assert bits & 1 and bits & 2
    got = ids.cpu().numpy()
    assert got.min() >= 0 and got.max() < SMALL.n_experts
    assert ctx.check_device_errors() == 0      # cleared


def _layer_case(moe, shape, cfg, T, flags=0, wts=None):
    wts = gpu_layer(shape, cfg, 0) if wts is None else wts
    ctx = moe.MoEContext(shape, n_layers=1, max_tokens=max(T, 1), flags=flags)
    ctx.register_layer(0, wts)
    x = fx.activations((cfg, "x", T), T, shape.hidden).numpy()
    xg = to_gpu(x)
    ids, w = ctx.route(0, xg)
    out = ctx.expert_forward(0, xg, ids, w)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    ref = ora.moe_layer(x, wts, shape)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref["ids"])
    assert_close(out.float().cpu().numpy(), ref["out"], f"{cfg} T={T}")
    ctx.close()
    return wts


@pytest.mark.parametrize("T", [1, 2, 7, 64])
def test_layer_small(moe, T):
    say(f"test_layer_small T={T}")
    _layer_case(moe, SMALL, "gpu-layer-small", T)


@pytest.mark.parametrize("T", [1, 16])
def test_layer_small_shared_renorm(moe, T):
    say(f"test_layer_small_shared_renorm T={T}")
    _layer_case(moe, SMALL_SHARED, "gpu-layer-shared", T)


@pytest.fixture(scope="module")
def olmoe_layer():
    return gpu_layer(fx.OLMOE, "olmoe-layer", 0)


@pytest.mark.parametrize("T", [4, 64, 512])
def test_layer_olmoe(moe, olmoe_layer, T):
    """OLMoE-shaped layer: decode T=4, batch-64 decode, 512-token prefill."""
    say(f"test_layer_olmoe T={T}")
    _layer_case(moe, fx.OLMOE, "olmoe-layer", T, wts=olmoe_layer)


def test_expert_forward_identical_experts_scale(moe):
    """All experts equal: out = (sum_j w) * FFN(x) on the GPU as well."""
    say("test_expert_forward_identical_experts_scale")
    wts = gpu_layer(SMALL, "gpu-ident", 0)
    for key in ("q", "s"):
        wts[key] = np.repeat(wts[key][:1], SMALL.n_experts, axis=0)
    _layer_case(moe, SMALL, "gpu-ident", 5, wts=wts)


def test_expert_forward_bad_ids_are_contained(moe):
    say("test_expert_forward_bad_ids_are_contained")
    wts = gpu_layer(SMALL, "gpu-badids", 0)
    ctx = _ctx(moe, SMALL)
    ctx.register_layer(0, wts)
    x = fx.activations(("badids",), 3, SMALL.hidden).cuda()
    ids = torch.tensor([[0, 1, 2, 3], [5, 5, 6, 7], [1, 2, 3, -4]], dtype=torch.int32, device="cuda")
    w = torch.full((3, 4), 0.25, dtype=torch.float32, device="cuda")
    out = ctx.expert_forward(0, x, ids, w)
    bits = ctx.check_device_errors()
    assert bits & 1 and bits & 2
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("T", [1, 5, 64])
@pytest.mark.parametrize("path", ["mfma", "gemv"])
def test_layer_small_forced_expert_path(moe, T, path):
    """Each expert path alone (MFMA grouped GEMM / INT4 GEMV) matches the oracle."""
    say(f"test_layer_small_forced_expert_path T={T} path={path}")
    flags = moe.MOE_FLAG_FORCE_MFMA if path == "mfma" else moe.MOE_FLAG_FORCE_GEMV
    _layer_case(moe, SMALL, "gpu-layer-small", T, flags=flags)
    _layer_case(moe, SMALL_SHARED, "gpu-layer-shared", T, flags=flags)


@pytest.mark.parametrize("T", [64, 512])
def test_layer_olmoe_forced_mfma(moe, olmoe_layer, T):
    say(f"test_layer_olmoe_forced_mfma T={T}")
    _layer_case(moe, fx.OLMOE, "olmoe-layer", T, flags=moe.MOE_FLAG_FORCE_MFMA, wts=olmoe_layer)


def _skewed_ids(T, E, k, heads, seed):
    """Forced routing with a few crowded experts: expert j of `heads` takes the
    first heads[j] tokens; the other slots of each token are distinct random
    experts from the rest."""
    rng = np.random.default_rng(seed)
    ids = np.zeros((T, k), dtype=np.int32)
    rest = np.arange(len(heads), E)
    for t in range(T):
        own = [j for j, c in enumerate(heads) if t < c][:k]
        fill = rng.choice(rest, k - len(own), replace=False)
        row = np.array(own + list(fill), dtype=np.int32)
        ids[t] = row[rng.permutation(k)]
    return ids


@pytest.mark.parametrize("shape_name", ["olmoe", "small"])
def test_layer_crowded_experts_mfma(moe, olmoe_layer, shape_name):
    """Grouped GEMM with token tiles of every size: an expert holding every
    token (several full 128-token tiles and a ragged one) and experts with
    120, 100, 90, 40, 20 and 5 tokens next to evenly spread ones.  The small
    shape runs the down projection with two weight sub-tiles per wave."""
    say(f"test_layer_crowded_experts_mfma {shape_name}")
    if shape_name == "olmoe":
        shape, wts, T = fx.OLMOE, olmoe_layer, 512
    else:
        shape, T = SMALL, 300
        wts = gpu_layer(shape, "gpu-crowded", 0)
    heads = [T, 120, 100, 90, 40, 20, 5][:shape.top_k]
    forced = _skewed_ids(T, shape.n_experts, shape.top_k, heads, 7)
    ctx = moe.MoEContext(shape, n_layers=1, max_tokens=T, flags=moe.MOE_FLAG_FORCE_MFMA)
    ctx.register_layer(0, wts)
    x = fx.activations(("crowded", shape_name), T, shape.hidden).numpy()
    xg = to_gpu(x)
    ids, w = ctx.route(0, xg, forced_ids=to_gpu(forced))
    out = ctx.expert_forward(0, xg, ids, w)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    ref = ora.moe_layer(x, wts, shape, forced_ids=forced)
    np.testing.assert_array_equal(ids.cpu().numpy(), forced)
    assert_close(out.float().cpu().numpy(), ref["out"], f"crowded {shape_name}")
    ctx.close()


def test_layer_crowded_experts_stream(moe, olmoe_layer):
    """Batched decode with skewed routing, all of it in the streaming kernel:
    experts with 64, 40 and 33 tokens (list entries of at most 32 tokens each:
    two, two and two), 32, 31 and 17 tokens (two 16-token sub-tiles) and 2 and
    1 (one sub-tile) next to evenly spread ones."""
    say("test_layer_crowded_experts_stream")
    shape, T = fx.OLMOE, 64
    heads = [64, 40, 33, 32, 31, 17, 2, 1]
    forced = _skewed_ids(T, shape.n_experts, shape.top_k, heads, 11)
    ctx = moe.MoEContext(shape, n_layers=1, max_tokens=T)
    ctx.register_layer(0, olmoe_layer)
    x = fx.activations(("crowded-stream",), T, shape.hidden).numpy()
    xg = to_gpu(x)
    ids, w = ctx.route(0, xg, forced_ids=to_gpu(forced))
    out = ctx.expert_forward(0, xg, ids, w)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    ref = ora.moe_layer(x, olmoe_layer, shape, forced_ids=forced)
    assert_close(out.float().cpu().numpy(), ref["out"], "crowded stream")
    ctx.close()


@pytest.mark.parametrize("case", ["ids_in_global", "masks_beyond_lds"])
def test_grouping_general_kernel_equals_one_pass(moe, case):
    """Batches too large for the one-pass grouping (more pairs than fit in LDS,
    or more (64-token chunk, expert) masks than fit) take the general grouping
    kernel.  A token's expert outputs do not depend on the other tokens of its
    tile, so the whole batch must equal its two halves (each grouped in one
    pass) bit for bit, on the grouped GEMM for both."""
    say(f"test_grouping_general_kernel_equals_one_pass {case}")
    if case == "ids_in_global":
        shape, T = SMALL, 4200  # 16,800 pairs
    else:
        shape, T = fx.MoEShape(hidden=256, n_experts=512, inter=256, top_k=8, renorm=False), 1024  # 16 x 512 masks
    wts = gpu_layer(shape, "gpu-group-general", 0)
    ctx = moe.MoEContext(shape, n_layers=1, max_tokens=T, flags=moe.MOE_FLAG_FORCE_MFMA)
    ctx.register_layer(0, wts)
    xg = to_gpu(fx.activations(("group-general", case), T, shape.hidden).numpy())
    ids, w = ctx.route(0, xg)
    whole = ctx.expert_forward(0, xg, ids, w).clone()
    h = T // 2
    first = ctx.expert_forward(0, xg[:h].contiguous(), ids[:h].contiguous(), w[:h].contiguous()).clone()
    second = ctx.expert_forward(0, xg[h:].contiguous(), ids[h:].contiguous(), w[h:].contiguous()).clone()
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    assert torch.equal(whole, torch.cat([first, second]))
    ctx.close()


@pytest.mark.parametrize("T", [17, 32])
def test_layer_shared_expert_two_subtiles(moe, T):
    """A shared expert that sees every token of a 17- or 32-token batch runs
    with two 16-token sub-tiles in the streaming kernel."""
    say(f"test_layer_shared_expert_two_subtiles T={T}")
    shape = fx.MoEShape(hidden=2048, n_experts=16, inter=512, top_k=2, renorm=True, shared_inter=512)
    _layer_case(moe, shape, "gpu-shared-2sub", T)


def test_boundary_rejects_empty_and_oversized_batches(moe):
    # T = 0 and T > max_tokens are refused before anything is enqueued, at every
    # entry point that takes a batch; the context keeps working afterwards
    import ctypes as C
    from w4a16_routed_expert_router_amd import capi
    say("test_boundary_rejects_empty_and_oversized_batches")
    wts = gpu_layer(SMALL, "gpu-boundary", 0)
    ctx = _ctx(moe, SMALL, max_tokens=8)
    ctx.register_layer(0, wts)
    lib, h = capi.load(), ctx._h
    H, k = SMALL.hidden, SMALL.top_k
    x = torch.zeros((16, H), dtype=torch.float16, device="cuda")
    hh = torch.zeros((16, H), dtype=torch.float32, device="cuda")
    ids = torch.zeros((16, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((16, k), dtype=torch.float32, device="cuda")
    out = torch.zeros((16, H), dtype=torch.float16, device="cuda")
    p = lambda t: C.c_void_p(t.data_ptr())
    for T in (0, 9, -1):
        assert lib.moe_route(h, 0, p(x), T, None, p(ids), p(w), None, None) == capi.MOE_E_ARG
        assert lib.moe_expert_forward(h, 0, p(x), T, p(ids), p(w), p(out), None) == capi.MOE_E_ARG
        assert lib.moe_stack_forward(h, 0, 1, p(hh), T, None, None, None, None, None) == capi.MOE_E_ARG
        assert lib.moe_rmsnorm(h, p(hh), T, p(out), None) == capi.MOE_E_ARG
        assert lib.moe_last_error(h)
    # an unregistered layer and a layer out of range are refused too
    assert lib.moe_route(h, 1, p(x), 1, None, p(ids), p(w), None, None) != capi.MOE_OK
    xs = fx.activations(("gpu-boundary-x",), 8, H).numpy()
    _check_route(ctx, wts, SMALL, xs)
    assert ctx.check_device_errors() == 0
    ctx.close()

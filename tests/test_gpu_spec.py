"""The opt-in batch-1 kernel that loads each layer's weights during the
previous layer (MOE_FLAG_GUESS_AHEAD): with the router's guess and with test
hooks that make the guess wrong for nearly every unit, for about half of them
or absent, every run equals the no-guess run bit for bit -- final residual and
every layer's x, ids and weights -- so the reload path and the matching of
units to guessed experts are exercised.  Each layer's routing equals the
oracle's routing of the kernel's own x, and the final residual matches the
oracle's stack within the layer tolerance whenever the routing agrees."""
import numpy as np
import pytest
import torch

from fixtures import moe_inputs as fx
from oracle import moe_oracle as ora

from gpu_util import assert_close, flip_is_explained, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import w4a16_routed_expert_router_amd as m
    return m


def _layers(shape, cfg, L):
    return [{k: v.cpu().numpy() for k, v in fx.layer_weights(shape, cfg, l, device="cuda", batched=True).items()}
            for l in range(L)]


# 128 experts: one logit replica per XCD holds 128 items, fewer than the 256
# exact and guess logits of a layer, so this shape runs on one replica
E128 = fx.MoEShape(hidden=2048, n_experts=128, inter=1024, top_k=8, renorm=True)


@pytest.mark.parametrize("shape_name,L", [("OLMOE", 16), ("QWEN_NEXT", 8), ("E128", 6)])
def test_speculative_weights_change_no_bit(moe, shape_name, L):
    say(f"test_speculative_weights_change_no_bit {shape_name} L={L}")
    shape = E128 if shape_name == "E128" else getattr(fx, shape_name)
    layers = _layers(shape, "spec-" + shape_name, L)
    ga = moe.capi.MOE_FLAG_GUESS_AHEAD
    modes = {"guess": ga, "none": ga | moe.capi.MOE_FLAG_TEST_GUESS_NONE,
             "lowest": ga | moe.capi.MOE_FLAG_TEST_GUESS_LOWEST, "shifted": ga | moe.capi.MOE_FLAG_TEST_GUESS_SHIFTED}
    runs = {}
    for name, flags in modes.items():
        ctx = moe.MoEContext(shape, n_layers=L, max_tokens=1, flags=flags)
        for l, w in enumerate(layers):
            ctx.register_layer(l, w)
        outs = []
        for i in range(3):
            h = torch.from_numpy(fx.activations(("spec", shape_name, i), 1, shape.hidden).numpy()
                                 .astype(np.float32)).cuda()
            xs, ids, ws = ctx.stack_forward(h, trace=True)
            torch.cuda.synchronize()
            outs.append((h.clone(), xs, ids, ws))
        assert ctx.check_device_errors() == 0
        ctx.close()
        runs[name] = outs
    for name in ("guess", "lowest", "shifted"):
        for i in range(3):
            for a, b in zip(runs[name][i], runs["none"][i]):
                assert torch.equal(a, b), (name, i)
    # and the path itself against the oracle: every layer's routing of the
    # kernel's own input, and the first input's final residual
    h0 = fx.activations(("spec", shape_name, 0), 1, shape.hidden).numpy()
    h, xs, ids, ws = runs["guess"][0]
    for l in range(L):
        o_ids, o_w, _ = ora.route(xs[l].cpu().numpy(), layers[l]["router"], shape.top_k, shape.renorm)
        np.testing.assert_array_equal(ids[l].cpu().numpy(), o_ids)
        np.testing.assert_allclose(ws[l].cpu().numpy(), o_w, rtol=1e-5, atol=1e-7)
    # the oracle's own free-running stack: equal routing gives the final
    # residual within tolerance; a routing difference must be a near-tie that
    # the drift between the two runs' inputs explains
    ref = ora.stack_forward(h0, layers, shape)
    for l in range(L):
        got = ids[l].cpu().numpy()[0]
        if not np.array_equal(got, ref["ids"][l][0]):
            ok, worst = flip_is_explained(xs[l].cpu().numpy()[0], ref["x"][l][0], layers[l]["router"],
                                          got, ref["ids"][l][0])
            say(f"  layer {l} routing differs from the oracle's run; margin {worst:.3e}")
            assert ok, (l, worst)
            return
    assert_close(h.cpu().numpy(), ref["h"], f"{shape_name} final h")

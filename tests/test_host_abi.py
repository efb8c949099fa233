"""Host-side checks of the HIP library that need no GPU: it loads, exports every
entry point the header declares, and its slot-pool decision engine makes the
same decisions as the oracle, event for event."""
import os
import re

import numpy as np
import pytest

from fixtures import moe_inputs as fx
from oracle import moe_oracle as ora

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4a16.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_hot_path_calls():
    names = _declared()
    for n in ("moe_create", "moe_destroy", "moe_register_layer", "moe_route",
              "moe_expert_forward", "moe_cache_ensure", "moe_stack_forward",
              "moe_cache_stats", "moe_cache_event_log"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from w4a16_routed_expert_router_amd import capi
    lib = capi.load()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(_declared()) == set(capi.SIGNATURES)


def test_create_rejects_bad_configs_without_touching_a_gpu():
    import ctypes as C
    from w4a16_routed_expert_router_amd import capi
    lib = capi.load()
    good = dict(hidden=2048, n_experts=64, inter=1024, top_k=8, renorm=0, n_layers=1,
                shared_inter=0, group=128, max_tokens=4, device=0, policy=0,
                slots_per_layer=0, flags=0)
    bad = [dict(hidden=100), dict(inter=4096), dict(top_k=0), dict(top_k=65, n_experts=64),
           dict(group=64), dict(max_tokens=0), dict(policy=7),
           dict(policy=1, slots_per_layer=4)]          # C < min(E, T*k) = 32
    for b in bad:
        cfg = capi.moe_config(**{**good, **b})
        h = C.c_void_p()
        st = lib.moe_create(C.byref(cfg), C.byref(h))
        assert st in (capi.MOE_E_SHAPE, capi.MOE_E_ARG, capi.MOE_E_CAPACITY), (b, st)
        assert not h.value
        assert lib.moe_last_error(None)


POLICY_NAMES = {ora.LRU: "lru", ora.LFU: "lfu", ora.LRU_FREQ: "lru_freq"}


@pytest.mark.parametrize("policy", [ora.LRU, ora.LFU, ora.LRU_FREQ])
@pytest.mark.parametrize("C", [8, 16, 32, 48])
def test_policy_engine_matches_oracle_on_zipf_trace(policy, C):
    from w4a16_routed_expert_router_amd import PolicyEngine
    trace = fx.zipf_trace("abi-zipf", 256, 2, 64, 8)
    for layer in range(2):
        sim = ora.CacheSim(policy, 64, C, layer=layer)
        eng = PolicyEngine(POLICY_NAMES[policy], 64, C, layer)
        for step in range(trace.shape[0]):
            g = trace[step, layer].tolist()
            want = sim.ensure(g, step)
            got = eng.access(g, step)
            assert got.tolist() == want
        assert eng.events() == [e.as_tuple() for e in sim.events]


@pytest.mark.parametrize("policy", [ora.LRU, ora.LFU, ora.LRU_FREQ])
def test_policy_engine_matches_oracle_on_unsorted_random_groups(policy):
    from w4a16_routed_expert_router_amd import PolicyEngine
    rng = np.random.default_rng(4)
    sim = ora.CacheSim(policy, 40, 10)
    eng = PolicyEngine(POLICY_NAMES[policy], 40, 10)
    for step in range(400):
        g = rng.choice(40, size=int(rng.integers(1, 11)), replace=False).tolist()
        assert eng.access(g, step).tolist() == sim.ensure(g, step)
    assert eng.events() == [e.as_tuple() for e in sim.events]


def test_policy_engine_rejects_bad_groups():
    from w4a16_routed_expert_router_amd import MoEError, PolicyEngine
    eng = PolicyEngine("lru", 8, 2)
    for g in ([1, 2, 3], [1, 1], [8], [-1]):
        with pytest.raises(MoEError):
            eng.access(g)
    assert eng.events() == []

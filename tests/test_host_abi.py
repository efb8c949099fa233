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
           dict(policy=1, slots_per_layer=4),          # C < min(E, T*k) = 32
           # staged transport without staging, or with fewer spare rows than
           # the misses one call can have (min(C, T*k) = 32): startup fails
           dict(policy=1, slots_per_layer=32, flags=16, staging_blobs=0, spare_rows=32),
           dict(policy=1, slots_per_layer=32, flags=16, staging_blobs=2, spare_rows=31),
           dict(policy=1, slots_per_layer=32, spare_rows=8),       # spare rows below 32
           dict(policy=1, slots_per_layer=32, spare_rows=-1)]
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


# ---- offline routing-trace analysis: native engine against the oracle -----------

def _oracle_groups(trace):
    """Rows of a [steps, width] trace as the oracle takes them: padding (< 0)
    dropped, repeats named once."""
    return [sorted(set(int(e) for e in row if e >= 0)) for row in trace]


def _mixed_trace(seed, steps, width, n_experts, pad_frac=0.15):
    rng = np.random.default_rng(seed)
    hot = rng.permutation(n_experts)[: max(2, n_experts // 4)]
    t = np.where(rng.random((steps, width)) < 0.6, rng.choice(hot, size=(steps, width)),
                 rng.integers(0, n_experts, size=(steps, width)))
    t[rng.random((steps, width)) < pad_frac] = -1
    return t.astype(np.int32)


@pytest.mark.parametrize("C", [8, 16, 32])
def test_trace_opt_and_policies_match_oracle_on_zipf_trace(C):
    import w4a16_routed_expert_router_amd as moe
    tr = fx.zipf_trace("abi-trace", 96, 2, 64, 8)
    for layer in range(2):
        rows = tr[:, layer, :]
        groups = _oracle_groups(rows)
        assert moe.trace_opt(rows, 64, C) == ora.opt_hits(groups, C)
        for pol in ("lru", "lfu", "lru_freq"):
            got = moe.trace_policy(pol, rows, 64, C)
            assert got == ora.policy_hits(pol, groups, 64, C)
            assert got[0] <= moe.trace_opt(rows, 64, C)[0]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_trace_analysis_matches_oracle_with_padding_and_repeats(seed):
    import w4a16_routed_expert_router_amd as moe
    E, width = 24, 6
    rows = _mixed_trace(seed, 80, width, E)
    groups = _oracle_groups(rows)
    for C in (width, 9, 16):
        assert moe.trace_opt(rows, E, C) == ora.opt_hits(groups, C)
        for pol in ("lru", "lfu", "lru_freq"):
            assert moe.trace_policy(pol, rows, E, C) == ora.policy_hits(pol, groups, E, C)
    for n_top in (0, 1, 3, E, E + 5):
        assert moe.trace_top_share(rows, E, n_top) == ora.top_share(ora.selection_counts(groups, E), n_top)
    got = moe.trace_skew(rows, E)
    want = ora.skew_report(groups, E)
    for key in ("top10", "top20", "top30"):
        assert got[key] == want[key]
    assert got["distinct"] == want["distinct"]
    assert got["selections"] == int(ora.selection_counts(groups, E).sum())
    assert abs(got["entropy_bits"] - want["entropy_bits"]) <= 1e-12 * max(1.0, want["entropy_bits"])


def test_trace_skew_matches_oracle_on_qwen_like_zipf_trace():
    import w4a16_routed_expert_router_amd as moe
    tr = fx.zipf_trace("abi-trace-qwen", 64, 1, 512, 10)[:, 0, :]
    groups = _oracle_groups(tr)
    got, want = moe.trace_skew(tr, 512), ora.skew_report(groups, 512)
    for key in ("top10", "top20", "top30", "distinct"):
        assert got[key] == want[key]
    assert abs(got["entropy_bits"] - want["entropy_bits"]) <= 1e-12 * want["entropy_bits"]
    assert moe.trace_opt(tr, 512, 40) == ora.opt_hits(groups, 40)


def test_trace_analysis_rejects_bad_traces():
    import w4a16_routed_expert_router_amd as moe
    from w4a16_routed_expert_router_amd import MoEError, capi
    rows = np.array([[0, 1, 2], [3, 4, 5]], dtype=np.int32)
    with pytest.raises(MoEError) as e:
        moe.trace_opt(rows, 5, 4)                 # id 5 out of range
    assert e.value.status == capi.MOE_E_ARG
    with pytest.raises(MoEError) as e:
        moe.trace_opt(rows, 8, 2)                 # a group of 3 in 2 slots
    assert e.value.status == capi.MOE_E_CAPACITY
    with pytest.raises(MoEError) as e:
        moe.trace_policy("lru", rows, 8, 2)
    assert e.value.status == capi.MOE_E_CAPACITY
    # an empty trace: nothing selected, no hits or misses
    empty = np.full((3, 4), -1, dtype=np.int32)
    assert moe.trace_opt(empty, 8, 1) == (0, 0)
    assert moe.trace_top_share(empty, 8, 2) == 0.0
    assert moe.trace_skew(empty, 8)["selections"] == 0


def _noisy_guess(rng, group, n_experts, p_wrong):
    """The next group with each expert replaced, with probability p_wrong, by a
    random expert not in it (a guess that is partly right)."""
    g = [int(e) for e in group]
    out = []
    for e in g:
        if rng.random() < p_wrong:
            cand = [x for x in range(n_experts) if x not in g and x not in out]
            out.append(int(rng.choice(cand)))
        else:
            out.append(e)
    return sorted(set(out))


@pytest.mark.parametrize("policy", ["lru", "lfu", "lru_freq"])
@pytest.mark.parametrize("C", [8, 16, 24])
def test_policy_engine_prefetch_matches_oracle(policy, C):
    from w4a16_routed_expert_router_amd import PolicyEngine
    rng = np.random.default_rng(C)
    tr = fx.zipf_trace("abi-prefetch", 120, 1, 64, 8)[:, 0, :]
    eng = PolicyEngine(policy, 64, C, layer=2)
    sim = ora.CacheSim(policy, 64, C, layer=2)
    for t in range(len(tr)):
        if t > 0 and rng.random() < 0.8:
            guess = _noisy_guess(rng, tr[t], 64, 0.3)
            eng.prefetch(guess, step=t)
            sim.prefetch(guess, step=t)
        eng.access(tr[t], step=t)
        sim.ensure(tr[t], step=t)
    assert eng.events() == [e.as_tuple() for e in sim.events]
    kinds = [e[3] for e in eng.events()]
    assert kinds.count(ora.EV_PREFETCH) == sim.prefetches > 0
    assert kinds.count(ora.EV_PREFETCH_HIT) == sim.prefetch_used > 0


def test_policy_engine_prefetch_rejects_bad_guesses():
    from w4a16_routed_expert_router_amd import MoEError, PolicyEngine, capi
    eng = PolicyEngine("lru", 16, 4)
    for bad, code in (([1, 1], capi.MOE_E_ARG), ([16], capi.MOE_E_ARG), ([0, 1, 2, 3, 4], capi.MOE_E_CAPACITY)):
        with pytest.raises(MoEError) as e:
            eng.prefetch(bad)
        assert e.value.status == code
    assert eng.events() == []


@pytest.mark.parametrize("policy", ["lru", "lfu", "lru_freq"])
def test_policy_engine_pin_matches_oracle(policy):
    from w4a16_routed_expert_router_amd import PolicyEngine
    rng = np.random.default_rng(7)
    tr = fx.zipf_trace("abi-pin", 100, 1, 64, 8)[:, 0, :]
    hot = sorted(int(e) for e in rng.choice(64, size=10, replace=False))
    eng = PolicyEngine(policy, 64, 20, layer=1)
    sim = ora.CacheSim(policy, 64, 20, layer=1)
    eng.pin(hot, step=0)
    sim.pin(hot, step=0)
    for t in range(len(tr)):
        if t and rng.random() < 0.5:
            guess = _noisy_guess(rng, tr[t], 64, 0.3)
            try:
                sim.prefetch(guess, step=t)
                eng.prefetch(guess, step=t)
            except ValueError:
                pass                                  # a guess that does not fit is refused by both
        eng.access(tr[t], step=t)
        sim.ensure(tr[t], step=t)
    assert eng.events() == [e.as_tuple() for e in sim.events]


@pytest.mark.parametrize("C,n_hot", [(16, 8), (24, 12), (32, 24)])
def test_trace_policy_pinned_matches_oracle(C, n_hot):
    import w4a16_routed_expert_router_amd as moe
    tr = fx.zipf_trace("abi-pin-trace", 96, 2, 64, 8)
    calib = fx.zipf_trace("abi-pin-calib", 96, 2, 64, 8)
    for layer in range(2):
        rows = tr[:, layer, :]
        groups = _oracle_groups(rows)
        cnt = ora.selection_counts(_oracle_groups(calib[:, layer, :]), 64)
        hot = sorted(sorted(range(64), key=lambda e: (-int(cnt[e]), e))[:n_hot])
        for pol in ("lru", "lfu", "lru_freq"):
            assert moe.trace_policy_pinned(pol, rows, 64, C, hot) == ora.policy_hits(pol, groups, 64, C, pinned=hot)


def test_pin_rejections():
    import w4a16_routed_expert_router_amd as moe
    from w4a16_routed_expert_router_amd import MoEError, PolicyEngine, capi
    eng = PolicyEngine("lru", 16, 4)
    for bad, code in (([1, 1], capi.MOE_E_ARG), ([16], capi.MOE_E_ARG), ([0, 1, 2, 3], capi.MOE_E_CAPACITY)):
        with pytest.raises(MoEError) as e:
            eng.pin(bad)
        assert e.value.status == code
    eng.access([5])
    with pytest.raises(MoEError) as e:
        eng.pin([1])                                   # not a cold pool
    assert e.value.status == capi.MOE_E_ARG
    eng2 = PolicyEngine("lfu", 16, 4)
    eng2.pin([0, 1])
    with pytest.raises(MoEError) as e:
        eng2.access([2, 3, 4])                         # three outside the hot set, two dynamic slots
    assert e.value.status == capi.MOE_E_CAPACITY
    eng2.access([0, 1, 2, 3])
    rows = np.array([[0, 1, 2]], dtype=np.int32)
    with pytest.raises(MoEError) as e:
        moe.trace_policy_pinned("lru", rows, 8, 3, [5, 6])   # 2 dynamic slots, 3 outside
    assert e.value.status == capi.MOE_E_CAPACITY

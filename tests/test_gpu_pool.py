"""Partial residency: an HBM expert-slot pool per layer backed by pinned host
memory.  Outputs must be bit-identical to full residency; hit/miss/eviction
sequences must equal the oracle's decisions; counters must add up."""
import numpy as np
import pytest
import torch

from fixtures import moe_inputs as fx
from oracle import moe_oracle as ora

from gpu_util import say

pytestmark = pytest.mark.gpu

L = 16
STEPS = 256
POLICY_ORACLE = {"lru": ora.LRU, "lfu": ora.LFU, "lru_freq": ora.LRU_FREQ}


@pytest.fixture(scope="module")
def moe():
    import w4a16_routed_expert_router_amd as m
    return m


@pytest.fixture(scope="module")
def olmoe_layers():
    return [{k: v.cpu().numpy() for k, v in
             fx.layer_weights(fx.OLMOE, "pool-olmoe", l, device="cuda", batched=True).items()}
            for l in range(L)]


@pytest.fixture(scope="module")
def trace():
    return fx.zipf_trace("pool-zipf", STEPS, L, fx.OLMOE.n_experts, fx.OLMOE.top_k, s=1.1)


@pytest.fixture(scope="module")
def h0s():
    return torch.stack([fx.activations(("pool-h0", i), 1, fx.OLMOE.hidden, device="cuda").float()
                        for i in range(32)])


def _ctx(moe, layers, **kw):
    ctx = moe.MoEContext(fx.OLMOE, n_layers=L, max_tokens=1, **kw)
    for l, w in enumerate(layers):
        ctx.register_layer(l, w)
    return ctx


def _run(ctx, trace, h0s, pooled, steps=STEPS, flags_check=True):
    outs = []
    ftr = torch.from_numpy(trace[:, :, None, :].copy()).cuda()     # [S, L, 1, k]
    for s in range(steps):
        if pooled:
            for l in range(L):
                ctx.cache_ensure(l, trace[s, l], step=s)
        h = h0s[s % len(h0s)].clone()
        ctx.stack_forward(h, forced_ids=ftr[s])
        outs.append(h)
    torch.cuda.synchronize()
    if flags_check:
        assert ctx.check_device_errors() == 0
    return torch.stack(outs)


@pytest.fixture(scope="module")
def resident_out(moe, olmoe_layers, trace, h0s):
    ctx = _ctx(moe, olmoe_layers)
    out = _run(ctx, trace, h0s, pooled=False)
    ctx.close()
    return out


@pytest.mark.parametrize("policy,C", [("lru", 16), ("lfu", 16), ("lfu", 32), ("lru", 48),
                                      ("lru_freq", 16)])
def test_pool_bit_identical_and_decisions_match_oracle(moe, olmoe_layers, trace, h0s,
                                                       resident_out, policy, C):
    say(f"test_pool policy={policy} C={C}")
    ctx = _ctx(moe, olmoe_layers, policy=policy, slots=C)
    out = _run(ctx, trace, h0s, pooled=True)
    assert torch.equal(out, resident_out), "cache changed the output"
    blob = fx.OLMOE.blob_bytes
    hit_rates = []
    for l in range(L):
        sim = ora.CacheSim(POLICY_ORACLE[policy], fx.OLMOE.n_experts, C, layer=l)
        for s in range(STEPS):
            sim.ensure(trace[s, l].tolist(), s)
        assert ctx.cache_events(l) == [e.as_tuple() for e in sim.events], f"layer {l}"
        st = ctx.cache_stats(l)
        assert st["accesses"] == STEPS * fx.OLMOE.top_k
        assert st["hits"] + st["misses"] == st["accesses"] and st["hits"] == sim.hits
        assert st["misses"] == sim.misses and st["h2d_bytes"] == sim.misses * blob
        assert st["evictions"] == sum(1 for e in sim.events if e.victim >= 0)
        assert st["d2h_bytes"] == 0 and st["failures"] == 0
        assert st["h2d_seconds"] > 0
        hit_rates.append(st["hits"] / st["accesses"])
    say(f"  mean hit rate {np.mean(hit_rates):.3f}")
    ctx.close()


def test_pool_transfer_failure_before_publication_keeps_state(moe, olmoe_layers, trace, h0s,
                                                              resident_out):
    say("test_pool_transfer_failure_before_publication_keeps_state")
    ctx = _ctx(moe, olmoe_layers, policy="lfu", slots=16)
    _run(ctx, trace, h0s, pooled=True, steps=10)
    before = ctx.cache_events(3), ctx.cache_stats(3)
    # a group of experts that are not resident after those 10 steps (all misses)
    sim = ora.CacheSim(ora.LFU, fx.OLMOE.n_experts, 16, layer=3)
    for s in range(10):
        sim.ensure(trace[s, 3].tolist(), s)
    miss_group = np.array([e for e in range(fx.OLMOE.n_experts) if e not in sim.slot_of][:8],
                          dtype=np.int32)
    ctx.inject_transfer_failure(3, 1)
    with pytest.raises(moe.MoEError) as ei:
        ctx.cache_ensure(3, miss_group, step=99)
    assert ei.value.status == 7          # MOE_E_TRANSFER
    after = ctx.cache_events(3), ctx.cache_stats(3)
    assert after[0] == before[0]
    assert after[1]["misses"] == before[1]["misses"] and after[1]["failures"] == 1
    # the context keeps working and stays exact
    ctx.cache_ensure(3, miss_group, step=99)
    ctx.close()


def test_pool_failure_after_publication_faults_context(moe, olmoe_layers):
    say("test_pool_failure_after_publication_faults_context")
    ctx = _ctx(moe, olmoe_layers, policy="lru", slots=16)
    ctx.inject_transfer_failure(0, 2)
    with pytest.raises(moe.MoEError) as ei:
        ctx.cache_ensure(0, np.arange(8, dtype=np.int32))
    assert ei.value.status == 8          # MOE_E_FAULTED
    with pytest.raises(moe.MoEError):
        ctx.cache_ensure(0, np.arange(8, dtype=np.int32))
    assert ctx.cache_stats(0)["failures"] == 1     # stats still readable
    ctx.close()


def test_pool_capacity_and_residency_errors(moe, olmoe_layers):
    say("test_pool_capacity_and_residency_errors")
    with pytest.raises(moe.MoEError) as ei:
        moe.MoEContext(fx.OLMOE, n_layers=1, max_tokens=4, policy="lru", slots=16)  # 4*8 > 16
    assert ei.value.status == 5
    ctx = _ctx(moe, olmoe_layers, policy="lru", slots=16)
    with pytest.raises(moe.MoEError) as ei:
        ctx.cache_ensure(0, np.arange(17, dtype=np.int32))
    assert ei.value.status == 5
    # running experts that were never made resident is contained and reported
    h = torch.zeros((1, fx.OLMOE.hidden), dtype=torch.float32, device="cuda")
    h[0, 0] = 1.0
    forced = torch.arange(8, dtype=torch.int32, device="cuda").reshape(1, 1, 8).repeat(L, 1, 1)
    ctx.stack_forward(h, forced_ids=forced)
    bits = ctx.check_device_errors()
    assert bits & 4
    ctx.close()


def test_pool_resident_all_ensure_is_identity(moe, olmoe_layers):
    ctx = _ctx(moe, olmoe_layers[:1] * L)
    g = np.array([5, 1, 9], dtype=np.int32)
    assert ctx.cache_ensure(0, g).tolist() == [5, 1, 9]
    assert ctx.cache_events(0) == []
    ctx.close()


# ---- natural routing over the pools, with and without next-layer prefetch ---------

NAT_STEPS = 12


def _run_natural(ctx, h0s, prefetch, steps=NAT_STEPS):
    outs, ids, gs = [], [], []
    for s in range(steps):
        h = h0s[s % len(h0s)].clone()
        i, g = ctx.stack_forward_pooled(h, step=s, prefetch=prefetch, trace=True)
        outs.append(h)
        ids.append(i.cpu().numpy())
        gs.append(g.cpu().numpy())
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    return torch.stack(outs), np.stack(ids), np.stack(gs)


def _replay(policy, C, ids, gs, prefetch, layer):
    """The oracle's decisions for one layer over the same routed groups and guesses."""
    sim = ora.CacheSim(POLICY_ORACLE[policy], fx.OLMOE.n_experts, C, layer=layer)
    for s in range(ids.shape[0]):
        if prefetch and layer > 0:
            guess = sorted(set(int(e) for e in gs[s, layer].ravel()))
            if len(guess) <= C:
                sim.prefetch(guess, s)
        sim.ensure(sorted(set(int(e) for e in ids[s, layer].ravel())), s)
    return sim


@pytest.mark.parametrize("policy,C", [("lru", 16), ("lfu", 32)])
def test_pool_natural_routing_prefetch_never_changes_outputs(moe, olmoe_layers, h0s, policy, C):
    say(f"test_pool_natural policy={policy} C={C}")
    runs = {}
    for pf in (False, True):
        ctx = _ctx(moe, olmoe_layers, policy=policy, slots=C)
        out, ids, gs = _run_natural(ctx, h0s, pf)
        blob = fx.OLMOE.blob_bytes
        used = issued = 0
        for l in range(L):
            sim = _replay(policy, C, ids, gs, pf, l)
            assert ctx.cache_events(l) == [e.as_tuple() for e in sim.events], f"layer {l} prefetch={pf}"
            st = ctx.cache_stats(l)
            assert st["hits"] == sim.hits and st["misses"] == sim.misses
            assert st["prefetches"] == sim.prefetches and st["prefetch_used"] == sim.prefetch_used
            assert st["h2d_bytes"] == (sim.misses + sim.prefetches) * blob
            assert st["d2h_bytes"] == 0 and st["failures"] == 0
            used += sim.prefetch_used
            issued += sim.prefetches
        if pf:
            assert issued > 0
            say(f"  prefetched {issued}, used {used} ({used / issued:.3f})")
        runs[pf] = (out, ids)
        ctx.close()
    # prefetching never changes what is computed
    assert torch.equal(runs[True][0], runs[False][0]), "prefetch changed the output"
    assert np.array_equal(runs[True][1], runs[False][1])


def test_pool_natural_routing_matches_resident_stack(moe, olmoe_layers, h0s):
    # the pooled per-layer loop against the whole-stack call with every expert
    # resident: the same routing on (nearly) the same x, outputs within tolerance
    from gpu_util import rel_l2
    ctx = _ctx(moe, olmoe_layers, policy="lru", slots=16)
    pooled, ids, _ = _run_natural(ctx, h0s, True, steps=4)
    ctx.close()
    ctx = _ctx(moe, olmoe_layers)
    for s in range(4):
        h = h0s[s].clone()
        _, rids, _ = ctx.stack_forward(h, trace=True)
        agree = float(np.mean(rids.cpu().numpy() == ids[s]))
        err = rel_l2(pooled[s].cpu().numpy(), h.cpu().numpy())
        say(f"  step {s}: ids agree {agree:.4f}, rel-L2 {err:.2e}")
        assert agree >= 0.99 and err <= 2e-3
    ctx.close()


def test_pool_prefetch_argument_errors(moe, olmoe_layers):
    from w4a16_routed_expert_router_amd import MoEError, capi
    ctx = _ctx(moe, olmoe_layers[:L], policy="lru", slots=8)
    for bad, code in (([3, 3], capi.MOE_E_ARG), ([64], capi.MOE_E_ARG), (list(range(9)), capi.MOE_E_CAPACITY)):
        with pytest.raises(MoEError) as e:
            ctx.cache_prefetch(1, bad)
        assert e.value.status == code
    assert ctx.cache_events(1) == []
    ctx.close()
    res = _ctx(moe, olmoe_layers)
    res.cache_prefetch(1, [1, 2, 3])      # full residency: nothing to do
    with pytest.raises(MoEError) as e:
        res.stack_forward_pooled(h=torch.zeros((1, fx.OLMOE.hidden), device="cuda"))
    assert e.value.status == capi.MOE_E_ARG
    res.close()


# ---- static / hybrid hot sets -------------------------------------------------------

def _hot_sets(n_hot):
    """Per layer, the n_hot most-selected experts of a calibration trace with the
    same popularity ranking as the test trace (other draws)."""
    calib = fx.zipf_trace("pool-zipf-calib", 128, L, fx.OLMOE.n_experts, fx.OLMOE.top_k, s=1.1,
                          perm_cfg="pool-zipf")
    hot = []
    for l in range(L):
        cnt = np.bincount(calib[:, l, :].ravel(), minlength=fx.OLMOE.n_experts)
        hot.append(sorted(sorted(range(fx.OLMOE.n_experts), key=lambda e: (-int(cnt[e]), e))[:n_hot]))
    return hot


@pytest.mark.parametrize("policy,C,n_hot", [("lfu", 24, 12), ("lru", 32, 20)])
def test_pool_hot_set_bit_identical_and_decisions_match_oracle(moe, olmoe_layers, trace, h0s, resident_out,
                                                              policy, C, n_hot):
    say(f"test_pool_hot_set policy={policy} C={C} hot={n_hot}")
    hot = _hot_sets(n_hot)
    ctx = _ctx(moe, olmoe_layers, policy=policy, slots=C)
    for l in range(L):
        ctx.cache_pin(l, hot[l], step=0)
    out = _run(ctx, trace, h0s, pooled=True)
    assert torch.equal(out, resident_out), "hot set changed the output"
    blob = fx.OLMOE.blob_bytes
    rates = []
    for l in range(L):
        sim = ora.CacheSim(POLICY_ORACLE[policy], fx.OLMOE.n_experts, C, layer=l)
        sim.pin(hot[l], 0)
        for s in range(STEPS):
            sim.ensure(trace[s, l].tolist(), s)
        assert ctx.cache_events(l) == [e.as_tuple() for e in sim.events], f"layer {l}"
        st = ctx.cache_stats(l)
        assert st["pinned"] == n_hot and st["hits"] == sim.hits and st["misses"] == sim.misses
        assert st["h2d_bytes"] == (sim.misses + n_hot) * blob
        rates.append(st["hits"] / st["accesses"])
    say(f"  mean hit rate {np.mean(rates):.3f}")
    # a pin is for a cold pool only
    from w4a16_routed_expert_router_amd import MoEError, capi
    with pytest.raises(MoEError) as e:
        ctx.cache_pin(0, [63])
    assert e.value.status == capi.MOE_E_ARG
    ctx.close()


# ---- staged transport: pageable source, pinned staging, spare rows, leases --------

STAGED = dict(flags=16, staging_blobs=2, spare_rows=8)
SPARE = dict(spare_rows=8)          # spare rows straight from the pinned backing


@pytest.mark.parametrize("policy,C,mode", [("lfu", 16, "staged"), ("lru_freq", 24, "staged"), ("lru", 16, "spare")])
def test_pool_staged_transport_bit_identical_and_decisions_match_oracle(moe, olmoe_layers, trace, h0s,
                                                                       resident_out, policy, C, mode):
    say(f"test_pool_staged policy={policy} C={C} mode={mode}")
    ctx = _ctx(moe, olmoe_layers, policy=policy, slots=C, **(STAGED if mode == "staged" else SPARE))
    out = _run(ctx, trace, h0s, pooled=True)
    assert torch.equal(out, resident_out), "staged transport changed the output"
    blob = fx.OLMOE.blob_bytes
    for l in range(L):
        sim = ora.CacheSim(POLICY_ORACLE[policy], fx.OLMOE.n_experts, C, layer=l)
        for s in range(STEPS):
            sim.ensure(trace[s, l].tolist(), s)
        assert ctx.cache_events(l) == [e.as_tuple() for e in sim.events], f"layer {l}"
        st = ctx.cache_stats(l)
        assert st["misses"] == sim.misses and st["h2d_bytes"] == sim.misses * blob and st["d2h_bytes"] == 0
    ctx.close()


def test_pool_staged_transport_natural_routing_prefetch_and_hot_set(moe, olmoe_layers, h0s):
    # natural routing with prefetch and a pinned hot set: the staged transport
    # gives the same bits and the same decisions as the pinned-backing one
    say("test_pool_staged_natural")
    hot = [sorted(range(4 * (l % 3), 4 * (l % 3) + 4)) for l in range(L)]
    res = {}
    for mode, kw in (("direct", {}), ("staged", STAGED), ("spare", SPARE)):
        ctx = _ctx(moe, olmoe_layers, policy="lru", slots=16, **kw)
        for l in range(L):
            ctx.cache_pin(l, hot[l])
        out, ids, gs = _run_natural(ctx, h0s, True)
        res[mode] = (out, ids, [ctx.cache_events(l) for l in range(L)])
        ctx.close()
    for mode in ("staged", "spare"):
        assert torch.equal(res[mode][0], res["direct"][0])
        assert np.array_equal(res[mode][1], res["direct"][1])
        assert res[mode][2] == res["direct"][2]


def test_pool_staged_transfer_failure_before_publication_keeps_state(moe, olmoe_layers, trace, h0s):
    say("test_pool_staged_transfer_failure")
    ctx = _ctx(moe, olmoe_layers, policy="lfu", slots=16, **STAGED)
    _run(ctx, trace, h0s, pooled=True, steps=10)
    sim = ora.CacheSim(ora.LFU, fx.OLMOE.n_experts, 16, layer=5)
    for s in range(10):
        sim.ensure(trace[s, 5].tolist(), s)
    miss_group = np.array([e for e in range(fx.OLMOE.n_experts) if e not in sim.slot_of][:8], dtype=np.int32)
    before = ctx.cache_events(5)
    ctx.inject_transfer_failure(5, 1)
    with pytest.raises(moe.MoEError) as ei:
        ctx.cache_ensure(5, miss_group, step=99)
    assert ei.value.status == 7          # MOE_E_TRANSFER: the old generation stays authoritative
    assert ctx.cache_events(5) == before
    ctx.cache_ensure(5, miss_group, step=99)
    sim.ensure(miss_group.tolist(), 99)
    assert ctx.cache_events(5) == [e.as_tuple() for e in sim.events]
    ctx.close()


def _chunks(ids_l, hot, dyn):
    """Greedy contiguous token chunks whose groups keep at most `dyn` experts
    outside the hot set (ids_l: [T, k] of one layer)."""
    out, t0, T = [], 0, ids_l.shape[0]
    grp = lambda a, b: sorted(set(int(e) for e in ids_l[a:b].ravel()))
    outside = lambda g: sum(1 for e in g if e not in hot)
    while t0 < T:
        t1 = t0 + 1
        while t1 < T and outside(grp(t0, t1 + 1)) <= dyn:
            t1 += 1
        out.append(grp(t0, t1))
        t0 = t1
    return out


def test_pool_batch_group_larger_than_dynamic_slots_runs_in_chunks(moe, olmoe_layers):
    # 4 tokens, C = 32 with 24 pinned: 8 dynamic slots, fewer than a 4-token
    # group usually needs, so layers run over token chunks; results equal the
    # all-resident stack's and decisions equal the oracle's over the same chunks
    say("test_pool_batch_group_chunks")
    from gpu_util import rel_l2
    T, C, n_hot, steps = 4, 32, 24, 6
    hot = _hot_sets(n_hot)
    ctx = moe.MoEContext(fx.OLMOE, n_layers=L, max_tokens=T, policy="lru", slots=C)
    for l, w in enumerate(olmoe_layers):
        ctx.register_layer(l, w)
        ctx.cache_pin(l, hot[l])
    res = moe.MoEContext(fx.OLMOE, n_layers=L, max_tokens=T)
    for l, w in enumerate(olmoe_layers):
        res.register_layer(l, w)
    sims = [ora.CacheSim(ora.LRU, fx.OLMOE.n_experts, C, layer=l) for l in range(L)]
    for l in range(L):
        sims[l].pin(hot[l], 0)
    n_chunked = 0
    for s in range(steps):
        h0 = fx.activations(("pool-chunks", s), T, fx.OLMOE.hidden, device="cuda").float()
        h = h0.clone()
        ids, gs = ctx.stack_forward_pooled(h, step=s, prefetch=True, trace=True)
        ids, gs = ids.cpu().numpy(), gs.cpu().numpy()
        hr = h0.clone()
        _, rids, _ = res.stack_forward(hr, trace=True)
        assert np.array_equal(rids.cpu().numpy(), ids)
        assert rel_l2(h.cpu().numpy(), hr.cpu().numpy()) <= 2e-3
        for l in range(L):
            if l > 0:
                guess = sorted(set(int(e) for e in gs[l].ravel()))
                try:
                    if len(guess) <= C:
                        sims[l].prefetch(guess, s)
                except ValueError:
                    pass                      # does not fit the dynamic slots: not prefetched
            chunks = _chunks(ids[l], set(hot[l]), C - n_hot)
            n_chunked += len(chunks) > 1
            for g in chunks:
                sims[l].ensure(g, s)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    assert n_chunked > 0
    for l in range(L):
        assert ctx.cache_events(l) == [e.as_tuple() for e in sims[l].events], f"layer {l}"
    say(f"  chunked layer calls: {n_chunked} of {steps * L}")
    ctx.close()
    res.close()


def test_pool_qwen_like_natural_routing_prefetch(moe):
    # the Qwen3-Next-like shape (512 experts, top-10 renormalised, always-on
    # shared expert outside the pool): natural routing over 64-slot pools with
    # prefetch gives the all-resident stack's ids and outputs, and the oracle's
    # decisions
    say("test_pool_qwen_like_natural_routing_prefetch")
    from gpu_util import rel_l2
    shape, nl, C, steps = fx.QWEN_NEXT, 4, 64, 6
    layers = [{k: v.cpu().numpy() for k, v in
               fx.layer_weights(shape, "pool-qwen", l, device="cuda", batched=True).items()}
              for l in range(nl)]
    pool = moe.MoEContext(shape, n_layers=nl, max_tokens=1, policy="lfu", slots=C, spare_rows=10)
    res = moe.MoEContext(shape, n_layers=nl, max_tokens=1)
    for l, w in enumerate(layers):
        pool.register_layer(l, w)
        res.register_layer(l, w)
    sims = [ora.CacheSim(ora.LFU, shape.n_experts, C, layer=l) for l in range(nl)]
    for s in range(steps):
        h0 = fx.activations(("pool-qwen-h0", s), 1, shape.hidden, device="cuda").float()
        h = h0.clone()
        ids, gs = pool.stack_forward_pooled(h, step=s, prefetch=True, trace=True)
        ids, gs = ids.cpu().numpy(), gs.cpu().numpy()
        hr = h0.clone()
        _, rids, _ = res.stack_forward(hr, trace=True)
        assert np.array_equal(rids.cpu().numpy(), ids)
        assert rel_l2(h.cpu().numpy(), hr.cpu().numpy()) <= 2e-3
        for l in range(nl):
            if l > 0:
                sims[l].prefetch(sorted(set(int(e) for e in gs[l].ravel())), s)
            sims[l].ensure(sorted(set(int(e) for e in ids[l].ravel())), s)
    torch.cuda.synchronize()
    assert pool.check_device_errors() == 0
    for l in range(nl):
        assert pool.cache_events(l) == [e.as_tuple() for e in sims[l].events], f"layer {l}"
        st = pool.cache_stats(l)
        assert st["prefetch_used"] == sims[l].prefetch_used
    pool.close()
    res.close()


# ---- publication ordering under delayed copies ----------------------------------
# Every host-to-device blob copy waits on the side stream before it starts, so a
# layer that read a slot without waiting for that slot's copy would read the row's
# previous occupant ("F51 Nitro / Nitro-MoE", "When forced on, the cache was slower
# - and once corrupt": a cache there corrupted outputs through an event-ordering
# mistake).  The wait is a bounded kernel; results must not change.
DELAY_US = 300
DELAY_STEPS = 48


@pytest.mark.parametrize("mode", ["in_place", "spare", "staged"])
def test_pool_delayed_copies_bit_identical(moe, olmoe_layers, trace, h0s, resident_out, mode):
    say(f"test_pool_delayed_copies mode={mode}")
    kw = {"in_place": {}, "spare": SPARE, "staged": STAGED}[mode]
    ctx = _ctx(moe, olmoe_layers, policy="lru", slots=16, **kw)
    ctx.delay_copies(DELAY_US)
    out = _run(ctx, trace, h0s, pooled=True, steps=DELAY_STEPS)
    assert torch.equal(out, resident_out[:DELAY_STEPS]), f"delayed copies changed the output ({mode})"
    for l in range(L):
        sim = ora.CacheSim(ora.LRU, fx.OLMOE.n_experts, 16, layer=l)
        for s in range(DELAY_STEPS):
            sim.ensure(trace[s, l].tolist(), s)
        assert ctx.cache_events(l) == [e.as_tuple() for e in sim.events], f"layer {l}"
        st = ctx.cache_stats(l)
        assert st["misses"] == sim.misses
        # the waits really ran: the side stream's busy time covers one per copy
        assert st["h2d_seconds"] >= 0.9 * sim.misses * DELAY_US * 1e-6, (l, st["h2d_seconds"], sim.misses)
    ctx.close()


def test_pool_delayed_copies_natural_routing_prefetch(moe, olmoe_layers, h0s):
    # next-layer prefetch and demand misses both delayed, with in-place slots and
    # spare rows: the same bits, ids and decisions as without the delay
    say("test_pool_delayed_copies_natural")
    for kw in ({}, SPARE):
        res = []
        for delay in (0, DELAY_US):
            ctx = _ctx(moe, olmoe_layers, policy="lfu", slots=16, **kw)
            ctx.delay_copies(delay)
            out, ids, _ = _run_natural(ctx, h0s, True, steps=24)
            res.append((out, ids, [ctx.cache_events(l) for l in range(L)]))
            ctx.close()
        assert torch.equal(res[0][0], res[1][0]), f"delayed copies changed the output {kw}"
        assert np.array_equal(res[0][1], res[1][1])
        assert res[0][2] == res[1][2]


def test_debug_delay_copies_argument_range(moe, olmoe_layers):
    from w4a16_routed_expert_router_amd import MoEError, capi
    ctx = _ctx(moe, olmoe_layers[:L], policy="lru", slots=8)
    for bad in (-1, capi.MOE_MAX_COPY_DELAY_US + 1):
        with pytest.raises(MoEError):
            ctx.delay_copies(bad)
    ctx.delay_copies(capi.MOE_MAX_COPY_DELAY_US)
    ctx.delay_copies(0)
    ctx.close()


def test_sync_each_call_reports_device_errors_at_the_call(moe, olmoe_layers, monkeypatch):
    # MOE_SYNC_EACH_CALL=1 (read when the context is created): the call that set
    # the device error word fails with MOE_E_DEVICE itself; without it the call
    # returns and the error shows at moe_check_device_errors.  Results are the
    # same either way.
    from w4a16_routed_expert_router_amd import MoEError, capi
    say("test_sync_each_call")
    shape = fx.OLMOE
    x = fx.activations(("sync-each",), 3, shape.hidden).cuda()
    bad = torch.tensor([[0, 1, 2, 3, 4, 5, 6, 7], [5, 5, 6, 7, 8, 9, 10, 11], [1, 2, 3, -4, 5, 6, 7, 8]],
                       dtype=torch.int32, device="cuda")
    w = torch.full((3, shape.top_k), 0.125, dtype=torch.float32, device="cuda")
    outs = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("MOE_SYNC_EACH_CALL", mode)
        ctx = moe.MoEContext(shape, n_layers=1, max_tokens=4)
        ctx.register_layer(0, olmoe_layers[0])
        ids, ww = ctx.route(0, x[:1])
        outs[mode] = ctx.expert_forward(0, x[:1], ids, ww).clone()
        if mode == "1":
            with pytest.raises(MoEError) as ei:
                ctx.expert_forward(0, x, bad, w)
            assert ei.value.status == capi.MOE_E_DEVICE
        else:
            ctx.expert_forward(0, x, bad, w)
        assert ctx.check_device_errors() & 3 == 3
        assert ctx.check_device_errors() == 0
        ctx.close()
    monkeypatch.delenv("MOE_SYNC_EACH_CALL")
    assert torch.equal(outs["0"], outs["1"])


# ---- two consumer streams ----------------------------------------------------------
@pytest.mark.parametrize("mode", ["in_place", "spare", "staged"])
def test_pool_two_consumer_streams_delayed_readers(moe, olmoe_layers, h0s, mode):
    """Two request streams on one pooled context ("Partial-residency contract:
    immutable authority and miss lifecycle": prior-generation consumers keep
    their leases; victim storage is reused only after they retire).  Requests
    alternate A, B; every A request starts with a ~1 ms spin on its stream, so
    its reads run late while B's ensures already transfer; copies are delayed
    too; with 12 slots for two groups of 8, B's misses evict experts that the
    pending A request reads.  Each stream's outputs equal a fully resident run
    of its own routing, bit for bit, and the decisions equal the oracle's over
    the interleaved groups."""
    say(f"test_pool_two_consumer_streams mode={mode}")
    # C < 2k: a B request's misses must evict experts of the A request just
    # before it, whose delayed reads are still pending
    steps, E, k, C = 24, fx.OLMOE.n_experts, fx.OLMOE.top_k, 12
    tr = {"A": fx.zipf_trace("pool-two-A", steps, L, E, k, s=1.1),
          "B": fx.zipf_trace("pool-two-B", steps, L, E, k, s=1.1)}
    res = _ctx(moe, olmoe_layers)
    ref = {n: _run(res, tr[n], h0s, pooled=False, steps=steps) for n in "AB"}
    res.close()
    kw = {"in_place": {}, "spare": SPARE, "staged": STAGED}[mode]
    ctx = _ctx(moe, olmoe_layers, policy="lru", slots=C, **kw)
    ctx.delay_copies(100)
    streams = {"A": torch.cuda.Stream(), "B": torch.cuda.Stream()}
    ftr = {n: torch.from_numpy(tr[n][:, :, None, :].copy()).cuda() for n in "AB"}
    torch.cuda.synchronize()
    outs = {"A": [], "B": []}
    for s in range(steps):
        for i, n in enumerate("AB"):
            st = streams[n]
            with torch.cuda.stream(st):
                if n == "A":
                    torch.cuda._sleep(2_000_000)
                for l in range(L):
                    ctx.cache_ensure(l, tr[n][s, l], step=2 * s + i, stream=st)
                h = h0s[s % len(h0s)].clone()
                ctx.stack_forward(h, forced_ids=ftr[n][s], stream=st)
                outs[n].append(h)
    torch.cuda.synchronize()
    assert ctx.check_device_errors() == 0
    for n in "AB":
        assert torch.equal(torch.stack(outs[n]), ref[n]), f"stream {n} output changed ({mode})"
    cross = 0  # B misses whose victim is an expert of the A request just before
    for l in range(L):
        sim = ora.CacheSim(ora.LRU, E, C, layer=l)
        for s in range(steps):
            sim.ensure(tr["A"][s, l].tolist(), 2 * s)
            n0 = len(sim.events)
            sim.ensure(tr["B"][s, l].tolist(), 2 * s + 1)
            cross += sum(1 for e in sim.events[n0:] if e.victim in set(tr["A"][s, l].tolist()))
        assert ctx.cache_events(l) == [e.as_tuple() for e in sim.events], f"layer {l}"
    say(f"  B misses evicting the pending A request's experts: {cross}")
    assert cross > 0
    ctx.close()

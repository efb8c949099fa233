#!/usr/bin/env python3
"""Benchmark: W4A16 MoE decode on an OLMoE-shaped 16-layer stack, batch 1.

Workload: 16 routed MoE layers (hidden 2048, 64 experts, intermediate 1024,
top-8, softmax without renormalisation, INT4 group-128 FP16 scales), RMSNorm
(eps 1e-5) between layers, no attention; all 1,024 experts resident in HBM.
32 seeded FP16 hidden states are processed one after another at batch 1; a
step is one token through all 16 layers (RMSNorm, router, grouping, gate/up +
SwiGLU, down, combine into the FP32 residual).  Inputs and weights are
resident in HBM before the timed region.

Prints one JSON line.  `value` is tokens/s through the whole stack.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
N_INPUTS = 32
N_CHECK = 4          # inputs whose final residual is checked against the oracle
REL_L2_TOL = 2e-3    # layer-output tolerance, applied to the final residual

# HBM bytes per launch of the fused decode kernel from the FETCH_SIZE /
# WRITE_SIZE counter passes (scaled by a 1 GiB reference copy), valid only for
# the kernel sources they were taken on (sha256 prefixes below); a changed
# kernel reports traffic = null until the counters are taken again.
COUNTED_TRAFFIC = {
    "bytes": 460_588_992,
    "sources": {"decode_fused.hip": "f3ac3570b7aa0ff2", "common.hpp": "bbd12f2f5f254678",
                "launch.hpp": "3d80c9ff07a13432", "fused_common.hpp": "a23f31d44a7efb9f",
                "exact_dot.hpp": "dd7ddc2f23467800", "topk_wave.hpp": "d6d1cd76583c6732"},
}


def counted_traffic():
    import hashlib
    csrc = os.path.join(ROOT, "w4a16_routed_expert_router_amd", "csrc")
    for name, want in COUNTED_TRAFFIC["sources"].items():
        with open(os.path.join(csrc, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != want:
                return None
    return COUNTED_TRAFFIC["bytes"]


# the other configurations and measurements, in the order they run
EXTRAS = {
    "olmoe_layer_t4": "extra_single_layer",
    "olmoe_layer_batched": "extra_batched",
    "qwen_next_like_stack": "extra_qwen",
    "partial_residency_olmoe16": "extra_pool",
    "prefetch_natural_routing_olmoe16": "extra_prefetch",
    "policy_sweep_zipf": "extra_trace_analysis",
}


def run_extra(name, moe, fx, dev, stream):
    fn = globals()[EXTRAS[name]]
    return fn(moe, fx) if name == "policy_sweep_zipf" else fn(moe, fx, dev, stream)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=320)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="wall-clock budget of the oracle's CPU baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", type=int, default=1, help="replay each step as a captured HIP graph")
    p.add_argument("--fused", type=int, default=1,
                   help="1: one persistent kernel per step; 0: per-layer kernels")
    p.add_argument("--extras", type=int, default=1,
                   help="1: also measure the batched (prefill / batch-64), Qwen-like and "
                        "partial-residency workloads, reported under \"extra\"")
    p.add_argument("--only", choices=sorted(EXTRAS), default=None,
                   help="run only this measurement (no headline line): prints its JSON and exits")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="run one device-to-device copy of this many MiB first (a reference "
                        "kernel of known traffic for hardware byte counters)")
    return p.parse_args()


def algorithmic_bytes_per_token(shape, n_layers):
    """Bytes a batch-1 token must read per stack pass: per layer the k routed
    experts' INT4 codes + FP16 scales and the FP16 router matrix."""
    per_layer = shape.top_k * shape.blob_bytes + shape.n_experts * shape.hidden * 2
    return n_layers * per_layer


def gateup_bytes_per_launch(shape, n_active):
    """Gate/up kernel: INT4 codes + scales of both matrices of each active expert."""
    return n_active * 2 * (shape.code_bytes + 2 * shape.scale_count)


def host_cpu():
    """CPU model (/proc/cpuinfo), the cores this process may run on, and the
    BLAS library numpy calls."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return model, cores, blas


def cpu_baseline(shape, layers_np, h0_np, budget_s, min_inputs):
    """The oracle on the host cores: as many whole 16-layer inputs as fit in
    `budget_s` (at least `min_inputs`), BLAS threads = the cores of the
    process's affinity mask."""
    from oracle import moe_oracle as ora
    model, cores, blas = host_cpu()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:
        limiter = None
    t0 = time.perf_counter()
    outs = []
    while len(outs) < len(h0_np):
        outs.append(ora.stack_forward(h0_np[len(outs)], layers_np, shape)["h"])
        if len(outs) >= min_inputs and time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    n = len(outs)
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} of the {len(h0_np)} batch-1 inputs through all {len(layers_np)} layers "
                      f"(float64 numpy oracle, exact router), {dt:.1f} s",
            "cpu": model, "blas": blas, "blas_threads": int(cores)}, outs


MFMA_FP16_PEAK_TFLOPS = 2500.0
N_REPLICAS = 4   # weight replicas rotated through so that 207.6 MB layers do not sit in the 256 MB MALL


def _rep_times_ms(fn, n, stream):
    """Per-call times (ms) of n calls, each between its own pair of events on
    `stream`; returns (median, p10, p90)."""
    import numpy as np
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    with torch.cuda.stream(stream):
        for i in range(n):
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
    ev[-1][1].synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def _event_time_ms(fn, n, stream):
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        a.record(stream)
        for i in range(n):
            fn(i)
        b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / n


def extra_single_layer(moe, fx, dev, stream, reps=100):
    """One OLMoE-shaped layer at 4 tokens, all 64 experts resident; weights rotate
    over 4 replicas (830 MB > MALL).  Two entry points: the layer calls
    (moe_route + moe_expert_forward: FP16 x in, FP16 out) and a one-layer
    moe_stack_forward (the one-launch kernel: RMSNorm, the layer and the FP32
    residual update, applied to the same residual call after call).  Per-call
    median and p10/p90 of `reps` calls each."""
    import numpy as np
    import torch
    shape, T = fx.OLMOE, 4
    ctx = moe.MoEContext(shape, n_layers=N_REPLICAS, max_tokens=T)
    for r in range(N_REPLICAS):
        w = fx.layer_weights(shape, "bench-layer-t4", r, device="cuda", batched=True)
        ctx.register_layer(r, {k: v.cpu().numpy() for k, v in w.items()})
        del w
    x = fx.activations(("bench-layer-t4-x",), T, shape.hidden, device="cuda")
    out = torch.empty_like(x)
    h0 = x.float()
    h = torch.empty_like(h0)
    ids_all = [ctx.route(r, x, stream=stream)[0] for r in range(N_REPLICAS)]
    stream.synchronize()
    used = float(np.mean([len(np.unique(i.cpu().numpy())) for i in ids_all]))
    nbytes = used * shape.blob_bytes + shape.n_experts * shape.hidden * 2 + 2 * T * shape.hidden * 2
    flops = 2.0 * T * shape.top_k * 3 * shape.hidden * shape.inter + 2.0 * T * shape.n_experts * shape.hidden

    def layer_api(i):
        r = i % N_REPLICAS
        ids, w = ctx.route(r, x, stream=stream)
        ctx.expert_forward(r, x, ids, w, out=out, stream=stream)

    def fused(i):
        # the layer reads the input residual from its own buffer and writes h
        # (moe_stack_forward_into: the timed region holds only the launch)
        r = i % N_REPLICAS
        ctx.stack_forward(h, layer_begin=r, layer_end=r + 1, h_in=h0, stream=stream)

    res = {"tokens": T, "experts_touched_mean": used, "bytes_per_call": int(nbytes), "flops_per_call": flops}
    for name, fn in (("layer_calls", layer_api), ("one_launch", fused)):
        for i in range(10):
            fn(i)
        med, p10, p90 = _rep_times_ms(fn, reps, stream)
        res[name] = {"us_median": round(med * 1e3, 2), "us_p10": round(p10 * 1e3, 2),
                     "us_p90": round(p90 * 1e3, 2), "tokens_per_s": round(T / (med * 1e-3), 1),
                     "hbm_gbps": round(nbytes / (med * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    assert ctx.check_device_errors(stream) == 0
    ctx.close()
    return res


def extra_batched(moe, fx, dev, stream):
    """One OLMoE-shaped layer (route + experts + combine) at 512-token prefill and
    batch-64 decode; router logits from the seeded FP16 router give the natural
    per-expert imbalance.  Weights rotate over 4 replicas (830 MB > MALL)."""
    import numpy as np
    import torch
    shape = fx.OLMOE
    ctx = moe.MoEContext(shape, n_layers=N_REPLICAS, max_tokens=512)
    for r in range(N_REPLICAS):
        w = fx.layer_weights(shape, "bench-batched", r, device="cuda", batched=True)
        ctx.register_layer(r, {k: v.cpu().numpy() for k, v in w.items()})
        del w
    res = {}
    for T, name in ((512, "prefill_512"), (64, "decode_batch64")):
        x = fx.activations(("bench-batched-x", T), T, shape.hidden, device="cuda")
        out = torch.empty_like(x)
        ids_w = [ctx.route(r, x, stream=stream) for r in range(N_REPLICAS)]
        stream.synchronize()

        def layer(i):
            r = i % N_REPLICAS
            ids, w = ctx.route(r, x, stream=stream)
            ctx.expert_forward(r, x, ids, w, out=out, stream=stream)

        for i in range(8):
            layer(i)
        ms = _event_time_ms(layer, 40, stream)
        # experts' part alone: the MFMA / GEMV expert kernels with ids fixed
        def experts(i):
            r = i % N_REPLICAS
            ids, w = ids_w[r]
            ctx.expert_forward(r, x, ids, w, out=out, stream=stream)
        ms_e = _event_time_ms(experts, 40, stream)
        counts = np.stack([np.bincount(ids.cpu().numpy().ravel(), minlength=shape.n_experts)
                           for ids, _ in ids_w])
        pairs = T * shape.top_k
        flops = 2.0 * pairs * 3 * shape.hidden * shape.inter + 2.0 * T * shape.n_experts * shape.hidden
        used = float(np.mean((counts > 0).sum(1)))
        nbytes = used * shape.blob_bytes + shape.n_experts * shape.hidden * 2 + T * shape.hidden * 4
        res[name] = {
            "tokens": T, "layer_us": round(ms * 1e3, 2), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "experts_us": round(ms_e * 1e3, 2),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_FP16_PEAK_TFLOPS, 4),
            "hbm_gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "tokens_per_expert_min_max": [int(counts.min()), int(counts.max())],
            "experts_used": used,
        }
    assert ctx.check_device_errors(stream) == 0
    ctx.close()
    return res


def extra_qwen(moe, fx, dev, stream, n_sets=8, n_layers=48, reps=50):
    """Qwen3-Next-like stack at its full 48 layers (512 experts, top-10
    renormalised, shared expert, I=512), decode at batch 1 and 16.  Layer l holds
    seeded weight set l % n_sets, each layer in storage of its own (39.9 GB of
    expert blobs stream every step).  Per-step median and p10/p90 of `reps`
    steps; bytes from the distinct experts each layer actually routes to."""
    import numpy as np
    import torch
    shape = fx.QWEN_NEXT
    res = {}
    ctx = moe.MoEContext(shape, n_layers=n_layers, max_tokens=16)
    sets = []
    for j in range(n_sets):
        w = fx.layer_weights(shape, "bench-qwen", j, device="cuda", batched=True)
        sets.append({k: v.cpu().numpy() for k, v in w.items()})
        del w
    for l in range(n_layers):
        ctx.register_layer(l, sets[l % n_sets])
    del sets
    blob_shared = shape.blob_bytes  # the shared expert has the routed shape
    router_b = shape.n_experts * shape.hidden * 2
    for T in (1, 16):
        h0 = fx.activations(("bench-qwen-h0", T), T, shape.hidden, device="cuda").float()
        h = torch.empty_like(h0)
        h.copy_(h0)
        _, ids, _ = ctx.stack_forward(h, trace=True, stream=stream)
        stream.synchronize()
        ids = ids.cpu().numpy()
        distinct = [len(np.unique(ids[l])) for l in range(n_layers)]
        nbytes = sum(u * shape.blob_bytes + blob_shared + router_b + 2 * T * shape.hidden * 4 for u in distinct)

        def step(i):
            ctx.stack_forward(h, h_in=h0, stream=stream)

        for i in range(5):
            step(i)
        med, p10, p90 = _rep_times_ms(step, reps, stream)
        res[f"batch_{T}"] = {
            "tokens": T, "layers": n_layers, "step_us_median": round(med * 1e3, 1),
            "step_us_p10": round(p10 * 1e3, 1), "step_us_p90": round(p90 * 1e3, 1),
            "per_layer_us": round(med * 1e3 / n_layers, 2),
            "tokens_per_s": round(T / (med * 1e-3), 1),
            "distinct_experts_per_layer_mean": round(float(np.mean(distinct)), 2),
            "bytes_per_step": int(nbytes),
            "hbm_gbps": round(nbytes / (med * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "path": "fused" if T <= 4 else "per-layer kernels"}
    assert ctx.check_device_errors(stream) == 0
    ctx.close()
    return res


def hbm_read_peak(stream, gib=2, n=10):
    """Measured HBM read-stream rate: a matrix-vector product (rocBLAS GEMV over
    the transposed view of a [8192, gib * 32768] FP32 matrix) that reads `gib`
    GiB once (beyond the 256 MB MALL) and writes 256 KiB; median of n runs.  Of
    the library routines tried it streamed fastest (torch.sum 4.0 TB/s, the
    untransposed GEMV 3.7)."""
    import torch
    with torch.cuda.stream(stream):
        a = torch.ones(8192, gib << 15, dtype=torch.float32, device="cuda")
        v = torch.ones(8192, dtype=torch.float32, device="cuda")
        y = torch.empty(gib << 15, dtype=torch.float32, device="cuda")
        for _ in range(2):
            torch.mv(a.t(), v, out=y)
    times = []
    for _ in range(n):
        times.append(_event_time_ms(lambda i: torch.mv(a.t(), v, out=y), 1, stream))
    del a
    return (gib << 30) / (sorted(times)[n // 2] * 1e-3) / 1e9


def pinned_h2d_peak(stream, nbytes, n=64):
    """Host -> device rate of n copies of `nbytes` from pinned memory on `stream`
    (the copy size of one OLMoE expert blob)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    with torch.cuda.stream(stream):
        for _ in range(4):
            dst.copy_(src, non_blocking=True)
    ms = _event_time_ms(lambda i: dst.copy_(src, non_blocking=True), n, stream)
    return nbytes / (ms * 1e-3) / 1e9


def extra_pool(moe, fx, dev, stream, steps=256, layers=16):
    """Partial residency on OLMoE shapes: per-layer HBM slot pools of C experts
    backed by pinned host copies of all 1,024 experts, routing forced by a seeded
    Zipf(1.1) popularity trace; hit rate, H2D traffic and tokens/s per policy and C,
    and bit-identity with full residency."""
    import numpy as np
    import torch
    shape = fx.OLMOE
    lw = [{k: v.cpu().numpy() for k, v in
           fx.layer_weights(shape, "bench-pool", l, device="cuda", batched=True).items()}
          for l in range(layers)]
    trace = fx.zipf_trace("bench-pool-zipf", steps, layers, shape.n_experts, shape.top_k, s=1.1)
    ftr = torch.from_numpy(trace[:, :, None, :].copy()).cuda()
    h0s = torch.stack([fx.activations(("bench-pool-h0", i), 1, shape.hidden, device="cuda").float()
                       for i in range(32)])

    def run(policy, C, **kw):
        ctx = moe.MoEContext(shape, n_layers=layers, max_tokens=1,
                             policy=policy, slots=C, **kw)
        for l, w in enumerate(lw):
            ctx.register_layer(l, w)
        outs = torch.empty((steps, 1, shape.hidden), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for s_ in range(steps):
                if policy != "resident":
                    for l in range(layers):
                        ctx.cache_ensure(l, trace[s_, l], step=s_, stream=stream)
                outs[s_].copy_(h0s[s_ % 32])
                ctx.stack_forward(outs[s_], forced_ids=ftr[s_], stream=stream)
        stream.synchronize()
        dt = time.perf_counter() - t0
        stats = [ctx.cache_stats(l) for l in range(layers)] if policy != "resident" else []
        assert ctx.check_device_errors(stream) == 0
        ctx.close()
        return outs, dt, stats

    ref, dt_ref, _ = run("resident", 0)
    peak = pinned_h2d_peak(stream, shape.blob_bytes)
    res = {"steps": steps, "layers": layers, "resident_tokens_per_s": round(steps / dt_ref, 1),
           "pinned_h2d_peak_gbps": round(peak, 2)}
    staged = dict(flags=moe.capi.MOE_FLAG_STAGED_TRANSPORT, staging_blobs=4, spare_rows=8)
    for policy, C, kw in (("lru", 16, {}), ("lfu", 16, {}), ("lru", 32, {}), ("lfu", 32, {}), ("lru", 48, {}),
                          ("lfu", 48, {}), ("lfu", 32, staged), ("lfu", 32, dict(spare_rows=8))):
        out, dt, st = run(policy, C, **kw)
        acc = sum(x["accesses"] for x in st)
        hits = sum(x["hits"] for x in st)
        h2d = sum(x["h2d_bytes"] for x in st)
        h2d_s = sum(x["h2d_seconds"] for x in st)
        res[f"{policy}_C{C}" + ("" if not kw else "_staged_transport" if "flags" in kw else "_spare_rows")] = {
            "hit_rate": round(hits / max(acc, 1), 4),
            "h2d_gb": round(h2d / 1e9, 3),
            "h2d_gbps_copy": round(h2d / max(h2d_s, 1e-12) / 1e9, 2),
            "h2d_copy_frac_of_pinned_peak": round(h2d / max(h2d_s, 1e-12) / 1e9 / peak, 3),
            "h2d_gbps_wall": round(h2d / dt / 1e9, 2),
            "tokens_per_s": round(steps / dt, 1),
            "bit_identical_to_resident": bool(torch.equal(out, ref)),
        }
    return res


def extra_prefetch(moe, fx, dev, stream, steps=64, layers=16):
    """Partial residency with natural routing (the router picks the experts; ids
    are read back per layer) on OLMoE shapes, batch 1, with and without
    next-layer prefetch (the next layer's router run on the current x guesses
    its experts, whose copies start while the current layer computes)."""
    import torch
    shape = fx.OLMOE
    lw = [{k: v.cpu().numpy() for k, v in
           fx.layer_weights(shape, "bench-prefetch", l, device="cuda", batched=True).items()}
          for l in range(layers)]
    h0s = torch.stack([fx.activations(("bench-prefetch-h0", i), 1, shape.hidden, device="cuda").float()
                       for i in range(32)])
    res = {"steps": steps, "layers": layers, "routing": "natural (router of each layer)"}
    for policy, C, spare in (("lru", 16, 0), ("lfu", 32, 0), ("lfu", 48, 0), ("lfu", 32, 8)):
        outs = {}
        for pf in (False, True):
            ctx = moe.MoEContext(shape, n_layers=layers, max_tokens=1, policy=policy, slots=C, spare_rows=spare)
            for l, w in enumerate(lw):
                ctx.register_layer(l, w)
            out = torch.empty((steps, 1, shape.hidden), dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            with torch.cuda.stream(stream):
                for s_ in range(steps):
                    out[s_].copy_(h0s[s_ % 32])
                    ctx.stack_forward_pooled(out[s_], step=s_, prefetch=pf, stream=stream)
            stream.synchronize()
            dt = time.perf_counter() - t0
            st = [ctx.cache_stats(l) for l in range(layers)]
            assert ctx.check_device_errors(stream) == 0
            ctx.close()
            acc = sum(x["accesses"] for x in st)
            pfs = sum(x["prefetches"] for x in st)
            row = {"tokens_per_s": round(steps / dt, 1),
                   "hit_rate": round(sum(x["hits"] for x in st) / max(acc, 1), 4),
                   "demand_misses_per_token": round(sum(x["misses"] for x in st) / steps, 2),
                   "h2d_gb": round(sum(x["h2d_bytes"] for x in st) / 1e9, 3)}
            if pf:
                row["prefetches_per_token"] = round(pfs / steps, 2)
                row["prefetch_used_frac"] = round(sum(x["prefetch_used"] for x in st) / max(pfs, 1), 4)
            outs[pf] = out
            tag = f"{policy}_C{C}" + (f"_spare{spare}" if spare else "")
            res[f"{tag}_{'prefetch' if pf else 'no_prefetch'}"] = row
        res[f"{tag}_bit_identical"] = bool(torch.equal(outs[True], outs[False]))
    return res


def hot_set_transfer(moe, fx, tr, E, k, C, steps, layers):
    """Hybrid pools (half the slots pinned to a hot set, the rest LFU) and static
    pools (all but k slots pinned) with the hot set calibrated on a trace with
    the same popularity ranking ("same prompt") or another one ("other
    prompt"); hit rates over the evaluation trace, means over layers."""
    import numpy as np
    same = fx.zipf_trace("bench-pool-zipf-calib", steps, layers, E, k, s=1.1, perm_cfg="bench-pool-zipf")
    other = fx.zipf_trace("bench-pool-zipf-other", steps, layers, E, k, s=1.1)
    accesses = steps * layers * k
    res = {}
    for n_hot, label in ((C // 2, "hybrid"), (C - k, "static")):
        if n_hot <= 0:
            continue
        for calib, cname in ((same, "same_prompt"), (other, "other_prompt")):
            h = 0
            for l in range(layers):
                cnt = np.bincount(calib[:, l, :].ravel(), minlength=E)
                hot = sorted(sorted(range(E), key=lambda e: (-int(cnt[e]), e))[:n_hot])
                h += moe.trace_policy_pinned("lfu", tr[:, l, :], E, C, hot)[0]
            res[f"{label}{n_hot}_lfu_{cname}_hit_rate"] = round(h / accesses, 4)
    return res


def extra_trace_analysis(moe, fx, steps=256):
    """Offline policy sweep over seeded Zipf(1.1) routing traces (host engine of the
    library): per capacity C the hit rates of LRU / LFU / LRU-FREQ and of Belady's
    OPT for groups, the gap to OPT, H2D copies per token, and the hit rate of a
    static pin of the C most-selected experts; per trace the top-10/20/30 % shares
    and the entropy of the selection frequencies (means over layers)."""
    import numpy as np
    res = {}
    for name, shape, layers, caps in (("olmoe16", fx.OLMOE, 16, (16, 32, 48, 64)),
                                      ("qwen_next_like48", fx.QWEN_NEXT, 48, (16, 32, 64, 128, 256))):
        E, k = shape.n_experts, shape.top_k
        tr = fx.zipf_trace("bench-pool-zipf" if name == "olmoe16" else "bench-qwen-zipf",
                           steps, layers, E, k, s=1.1)
        accesses = steps * layers * k
        sk = [moe.trace_skew(tr[:, l, :], E) for l in range(layers)]
        out = {"steps": steps, "layers": layers, "experts": E, "top_k": k,
               "skew": {key: round(float(np.mean([r[key] for r in sk])), 4)
                        for key in ("top10", "top20", "top30", "entropy_bits")}}
        out["skew"]["entropy_uniform_bits"] = round(float(np.log2(E)), 4)
        for C in caps:
            row = {}
            tot = {}
            for pol in ("lru", "lfu", "lru_freq", "opt"):
                h = m = 0
                for l in range(layers):
                    hh, mm = (moe.trace_opt(tr[:, l, :], E, C) if pol == "opt"
                              else moe.trace_policy(pol, tr[:, l, :], E, C))
                    h += hh
                    m += mm
                tot[pol] = (h, m)
                row[f"{pol}_hit_rate"] = round(h / accesses, 4)
            for pol in ("lru", "lfu", "lru_freq"):
                row[f"{pol}_gap_to_opt"] = round((tot["opt"][0] - tot[pol][0]) / accesses, 4)
                row[f"{pol}_h2d_copies_per_token"] = round(tot[pol][1] / steps, 2)
            row["opt_h2d_copies_per_token"] = round(tot["opt"][1] / steps, 2)
            row["static_pin_hit_rate"] = round(float(np.mean(
                [moe.trace_top_share(tr[:, l, :], E, C) for l in range(layers)])), 4)
            if name == "olmoe16" and C < E:
                row.update(hot_set_transfer(moe, fx, tr, E, k, C, steps, layers))
            out[f"C{C}"] = row
        res[name] = out
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1 "
                          "(expert-parallel sharding over several GPUs is not built)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import w4a16_routed_expert_router_amd as moe
    from fixtures import moe_inputs as fx

    shape, L, T = fx.OLMOE, 16, 1
    dev = torch.device("cuda", 0)
    # one stream for everything: inputs, library calls, copies and checks are
    # all ordered on it (graph capture needs a stream other than the default)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 18          # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {args.copy_calibration_mib} MiB read + "
              f"{args.copy_calibration_mib} MiB written", file=sys.stderr, flush=True)
        del src, dst
    if args.only:
        res = run_extra(args.only, moe, fx, dev, stream)
        print(json.dumps({"workload": args.only, "result": res}))
        return
    t_gen = time.perf_counter()
    ctx = moe.MoEContext(shape, n_layers=L, max_tokens=T,
                         flags=0 if args.fused else moe.MOE_FLAG_NO_FUSED)
    layers_np = []
    for layer in range(L):
        w = fx.layer_weights(shape, "bench-olmoe-stack", layer, device="cuda", batched=True)
        wn = {k: v.cpu().numpy() for k, v in w.items()}
        del w
        ctx.register_layer(layer, wn)
        layers_np.append(wn)
    h0 = torch.stack([fx.activations(("bench-h0", i), T, shape.hidden, device="cuda").float()
                      for i in range(N_INPUTS)])
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] weights generated and registered in {t_gen:.1f} s", file=sys.stderr, flush=True)

    h = torch.empty((T, shape.hidden), dtype=torch.float32, device=dev)

    # one step: the token's input residual (resident, in its own buffer) through
    # all layers into h (moe_stack_forward_into: one kernel, no copy first)
    def step(i):
        ctx.stack_forward(h, h_in=h0[i % N_INPUTS], stream=stream)

    graphs = None
    if args.graph:
        graphs = []
        with torch.cuda.stream(stream):
            for i in range(2):              # warm both code paths before capture
                step(i)
        stream.synchronize()
        # one graph per input slot keeps the input buffer fixed inside the graph
        for i in range(N_INPUTS):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(i)
            graphs.append(g)

    def run(i):
        if graphs is not None:
            with torch.cuda.stream(stream):
                graphs[i % N_INPUTS].replay()
        else:
            with torch.cuda.stream(stream):
                step(i)

    for i in range(args.warmup):
        run(i)
    stream.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    stream.synchronize()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    tok_s = T * args.steps / dt

    # dominant kernel, timed with HIP events on the stream it runs on: the fused
    # decode kernel (one launch = all 16 layers of a step) when the step takes
    # the fused path, else the gate/up kernel
    kind = "fused" if args.fused else "gateup"
    ctx.timer_enable(kind)
    ctx.timer_read()
    kt_steps = min(args.steps, 2 * N_INPUTS)
    with torch.cuda.stream(stream):
        for i in range(kt_steps):
            step(i)
    stream.synchronize()
    total_ms, launches = ctx.timer_read()
    ctx.timer_enable(None)
    avg_ms = total_ms / max(launches, 1)
    if kind == "fused":
        kname, per_launch = "fused_decode_kernel<2048,1024>", algorithmic_bytes_per_token(shape, L) * T
    else:
        kname, per_launch = "gateup_gemv_kernel<64>", gateup_bytes_per_launch(shape, shape.top_k * T)
    achieved = per_launch / (avg_ms * 1e-3) / 1e9

    # final residuals of the first inputs, compared with the oracle below: the
    # graph replays the timed loop ran, and direct launches.  Every copy is
    # enqueued on `stream`, the stream the kernel runs on, so nothing reads
    # an input before it has landed.
    finals_graph, finals_direct = [], []
    with torch.cuda.stream(stream):
        for i in range(N_CHECK):
            run(i)
            finals_graph.append(h.clone())
            hb = h0[i].clone()
            ctx.stack_forward(hb, stream=stream)
            finals_direct.append(hb)
    stream.synchronize()
    graph_eq_direct = all(torch.equal(a, b) for a, b in zip(finals_graph, finals_direct))
    assert ctx.check_device_errors(stream) == 0

    bytes_tok = algorithmic_bytes_per_token(shape, L)
    read_peak = hbm_read_peak(stream)
    out = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (W4A16 decode), OLMoE/Qwen-Next shapes",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dt / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "olmoe-16-layer-moe-stack-decode-batch1",
                   "hidden": shape.hidden, "experts": shape.n_experts, "inter": shape.inter,
                   "top_k": shape.top_k, "layers": L, "batch": T, "inputs": N_INPUTS,
                   "weights": "int4 g128 fp16 scales", "graph": bool(args.graph),
                   "fused": bool(args.fused)},
        "hbm_gbps_algorithmic": round(bytes_tok * tok_s / 1e9, 1),
        "bytes_per_token": bytes_tok,
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": counted_traffic() if kind == "fused" else None,
                     "bytes_per_launch": per_launch, "avg_launch_us": round(avg_ms * 1e3, 3),
                     "launches": launches,
                     "frac_of_measured_read_peak": round(achieved / read_peak, 4)},
        "hbm_read_peak_measured": {"gbps": round(read_peak, 1),
                                   "how": "GEMV reading 2 GiB of FP32 once (torch.mv on a transposed view), timed stream, median of 10"},
    }
    if args.extras:
        stream.synchronize()
        extra = {}
        t_x = time.perf_counter()
        for name in EXTRAS:
            extra[name] = run_extra(name, moe, fx, dev, stream)
            print(f"[bench] {name} done ({time.perf_counter() - t_x:.1f} s)", file=sys.stderr, flush=True)
        out["extra"] = extra
    # the oracle: the CPU baseline (timed) and the reference of the check;
    # with --no-cpu-baseline only the checked inputs are computed, untimed
    h0_np = [h0[i].cpu().numpy().astype(np.float16) for i in range(N_INPUTS)]
    if not args.no_cpu_baseline:
        cb, refs = cpu_baseline(shape, layers_np, h0_np, args.cpu_seconds, N_CHECK)
        out["cpu_baseline"] = cb
    else:
        from oracle import moe_oracle as ora
        refs = [ora.stack_forward(h0_np[i], layers_np, shape)["h"] for i in range(N_CHECK)]
    errs = []
    for i in range(N_CHECK):
        ref = refs[i]
        for got_t in (finals_graph[i], finals_direct[i]):
            got = got_t.cpu().numpy().astype(np.float64).reshape(ref.shape)
            errs.append(float(np.linalg.norm(got - ref) / np.linalg.norm(ref)))
    ok = graph_eq_direct and max(errs) <= REL_L2_TOL
    out["oracle_check"] = {"inputs": N_CHECK, "checked": "graph replays of the timed loop and direct launches",
                           "max_rel_l2": max(errs), "tolerance": REL_L2_TOL,
                           "graph_equals_direct": graph_eq_direct, "pass": ok}
    if not ok:
        out["valid"] = False
    print(json.dumps(out), flush=True)
    ctx.close()
    if not out["oracle_check"]["pass"]:
        print("[bench] oracle check FAILED: the timed path's outputs disagree with the oracle",
              file=sys.stderr, flush=True)
        sys.exit(3)


if __name__ == "__main__":
    main()

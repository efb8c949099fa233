"""CPU oracle for the W4A16 routed-expert MoE layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

It is a plain, slow, obviously correct statement of what the layer computes,
in float64 (plus one exact-integer step for the router), written from these
web pages:

  [HR]  "Horizon RunMap - Architecture, Results and Public Evaluation"
        (sections "Architecture invariants", "What is implemented",
        "The complete execution path", "Representation and computation",
        "Partial-residency contract: immutable authority and miss lifecycle")
  [MS]  "An expert-offloading engine, from scratch" (moe-stream; "Terms used
        here", "What the numbers say", "Correct first")
  [F51] "F51 Nitro / Nitro-MoE" ("The thesis", "Layer 1 - expert persistence
        cache", "The simulator")

Readings taken where the pages are silent are stated at each function.
Parity status: every function here is pinned by tests/test_oracle_pins.py
(closed forms, brute force, exact arithmetic) except where a docstring says
"parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

RMS_EPS = 1e-5

# ----------------------------------------------------------------------------
# INT4 weights with FP16 group scales  ([HR] "Architecture invariants": routed
# experts are kept as INT4 packed data with FP16 scales; "What is implemented":
# they stay compact on the GPU and are never persisted as expanded matrices).
# ----------------------------------------------------------------------------


def unpack_int4(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    """Packed bytes [n, k/2] -> codes int64 [n, k] in 0..15.

    Canonical layout: element 2j of a row sits in the low nibble of byte j,
    element 2j+1 in the high nibble.
    """
    b = np.asarray(packed, dtype=np.uint8).reshape(n, k // 2).astype(np.int64)
    codes = np.empty((n, k), dtype=np.int64)
    codes[:, 0::2] = b & 0xF
    codes[:, 1::2] = b >> 4
    return codes


def dequantize(packed: np.ndarray, scales: np.ndarray, n: int, k: int, group: int = 128) -> np.ndarray:
    """W[n, k] = (q[n, k] - 8) * s[n, k // group], in float64 (exact: a 4-bit
    integer times an FP16 value needs at most 15 significant bits)."""
    q = unpack_int4(packed, n, k)
    s = np.asarray(scales, dtype=np.float16).reshape(n, k // group).astype(np.float64)
    return (q - 8).astype(np.float64) * np.repeat(s, group, axis=1)


def expert_matrices(q: np.ndarray, s: np.ndarray, hidden: int, inter: int, group: int = 128):
    """One expert's dequantised (gate [I,H], up [I,H], down [H,I]) from its
    packed codes q [3, I*H/2] and scales s [3, I*H/group]."""
    H, I = hidden, inter
    gate = dequantize(q[0], s[0], I, H, group)
    up = dequantize(q[1], s[1], I, H, group)
    down = dequantize(q[2], s[2], H, I, group)
    return gate, up, down


# ----------------------------------------------------------------------------
# Router ([HR] "The complete execution path", step 2: each token is routed to
# its selected experts; [MS] "Terms used here": a router picks 8 of 64 experts
# per token at each of 16 layers; [F51] "The thesis": 10 of 512 plus a shared
# expert).  The router matrix is a non-routed FP16 weight ([HR] "Architecture
# invariants").
#
# Reading (the pages do not say how logits are summed): logit[t, e] is the
# FP32 value nearest (ties to even) to the EXACT real sum sum_i x[t,i]*Wr[e,i]
# of the FP16 inputs.  This makes the logits -- and therefore the selected
# experts -- independent of summation order.
# ----------------------------------------------------------------------------


def fp16_as_int(a) -> np.ndarray:
    """Every finite FP16 value is an integer multiple of 2^-24; return that
    integer (|X| < 2^40) as int64."""
    a64 = np.asarray(a, dtype=np.float16).astype(np.float64)
    if not np.all(np.isfinite(a64)):
        raise ValueError("non-finite FP16 input")
    return (a64 * 2.0 ** 24).astype(np.int64)


def exact_dot_ints(xi: np.ndarray, wi: np.ndarray) -> np.ndarray:
    """Exact integer dot products S[t, e] = sum_i xi[t,i] * wi[e,i] as Python ints.

    Each |value| < 2^40 is split as v = vh*2^20 + vl with vl in [0, 2^20), so
    every partial product is below 2^40 in magnitude and every int64 matmul
    over H <= 2^22 terms stays below 2^62: all four products are exact.
    """
    xi = np.asarray(xi, dtype=np.int64)
    wi = np.asarray(wi, dtype=np.int64)
    assert xi.shape[-1] == wi.shape[-1] and xi.shape[-1] <= (1 << 22)
    xh = xi >> 20
    xl = xi - (xh << 20)
    wh = wi >> 20
    wl = wi - (wh << 20)
    hh = (xh @ wh.T).astype(object)
    mid = (xh @ wl.T).astype(object) + (xl @ wh.T).astype(object)
    ll = (xl @ wl.T).astype(object)
    return hh * (1 << 40) + mid * (1 << 20) + ll


def round_int_scaled_to_f32(S: int, exp2: int) -> np.float32:
    """The FP32 value nearest to S * 2^exp2 (S a Python int), ties to even.

    Valid while the result is a normal FP32 number or zero, which holds for
    every dot product of FP16 vectors of length <= 2^22 (|value| <= 2^54 and
    any nonzero value is >= 2^-48).
    """
    if S == 0:
        return np.float32(0.0)
    neg = S < 0
    m = -S if neg else S
    nb = m.bit_length()
    shift = nb - 24
    if shift > 0:
        q, r = divmod(m, 1 << shift)
        half = 1 << (shift - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
        m, e = q, exp2 + shift          # q may be 2^24: still exact below
    else:
        e = exp2
    v = math.ldexp(float(m), e)         # m < 2^25: exact in float64
    out = np.float32(v)                 # exact: v has <= 24 significant bits
    assert float(out) == v
    return np.float32(-out) if neg else out


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """FP32 logits [T, E] = correctly rounded exact dot products of FP16 x [T, H]
    and FP16 router rows wr [E, H]."""
    S = exact_dot_ints(fp16_as_int(x), fp16_as_int(wr))
    out = np.empty(S.shape, dtype=np.float32)
    for idx in np.ndindex(S.shape):
        out[idx] = round_int_scaled_to_f32(int(S[idx]), -48)
    return out


def softmax(logits: np.ndarray) -> np.ndarray:
    """Softmax over experts of FP32 logits, in float64 (max-subtracted)."""
    z = np.asarray(logits, dtype=np.float64)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """The k experts with the largest logits, in rank order, ties to the lowest
    expert id: sort by (logit descending, id ascending) and keep the first k.
    Selection uses the logits, not the probabilities."""
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    eid = np.arange(E)
    for t in range(T):
        order = np.lexsort((eid, -logits[t].astype(np.float64)))
        ids[t] = order[:k]
    return ids


def combine_weights(p: np.ndarray, ids: np.ndarray, renorm: bool) -> np.ndarray:
    """w[t, j] = p[t, ids[t, j]]; renormalised over the chosen experts when
    `renorm` (Qwen3-Next-style layers), left as softmax probabilities otherwise
    (OLMoE-style layers)."""
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def route(x: np.ndarray, wr: np.ndarray, k: int, renorm: bool, forced_ids=None):
    """Router step: (ids int32 [T,k], w float64 [T,k], logits fp32 [T,E]).

    With `forced_ids` (a routing trace, [T, k]) the selection is skipped and
    the softmax probabilities are gathered at the forced experts, so a
    popularity trace can drive which experts run while the weights still come
    from this layer's router."""
    logits = router_logits(x, wr)
    p = softmax(logits)
    ids = topk(logits, k) if forced_ids is None else np.asarray(forced_ids, dtype=np.int32)
    return ids, combine_weights(p, ids, renorm), logits


# ----------------------------------------------------------------------------
# Expert FFN and combine ([HR] "The complete execution path", step 2: custom
# W4A16 kernels run the selected experts from compact weights with FP16
# activations).  SwiGLU with SiLU on the gate branch is the plain reading.
# ----------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def expert_ffn(x: np.ndarray, gate: np.ndarray, up: np.ndarray, down: np.ndarray) -> np.ndarray:
    """y = (silu(x gate^T) * (x up^T)) down^T for rows x [n, H] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ gate.T
    u = x @ up.T
    return (silu(g) * u) @ down.T


def moe_layer(x: np.ndarray, weights: dict, shape, forced_ids=None) -> dict:
    """One MoE layer on FP16 tokens x [T, H].

    weights: numpy arrays router fp16 [E,H], q uint8 [E,3,I*H/2],
    s fp16 [E,3,I*H/128] (+ shared_q, shared_s when the layer has a shared
    expert).  Returns ids, w, logits and out (float64 [T, H]) where
    out[t] = sum_{j=0}^{k-1} w[t,j] * FFN_{ids[t,j]}(x[t]) summed in rank
    order, plus FFN_shared(x[t]) with weight 1 when a shared expert exists.
    Each touched expert is dequantised once per call.
    """
    H, I, g = shape.hidden, shape.inter, shape.group
    x = np.asarray(x, dtype=np.float16)
    T = x.shape[0]
    ids, w, logits = route(x, weights["router"], shape.top_k, shape.renorm, forced_ids)
    x64 = x.astype(np.float64)
    y = np.zeros((T, shape.top_k, H), dtype=np.float64)
    for e in np.unique(ids):
        rows = np.argwhere(ids == e)                 # (t, j) pairs routed to e
        mats = expert_matrices(weights["q"][e], weights["s"][e], H, I, g)
        y[rows[:, 0], rows[:, 1]] = expert_ffn(x64[rows[:, 0]], *mats)
    out = np.zeros((T, H), dtype=np.float64)
    for j in range(shape.top_k):
        out += w[:, j:j + 1] * y[:, j]
    if shape.shared_inter:
        mats = expert_matrices(weights["shared_q"], weights["shared_s"], H, shape.shared_inter, g)
        out += expert_ffn(x64, *mats)
    return {"ids": ids, "w": w, "logits": logits, "out": out}


# ----------------------------------------------------------------------------
# Stacks of MoE layers.  The pages' models run 16 (OLMoE, [MS] "Terms used
# here") or 48 ([F51] "The thesis") routed layers.  Reading: a pre-norm
# residual stack without attention, h <- h + MoE_l(fp16(RMSNorm(h))), RMSNorm
# with unit weight and eps 1e-5, residual kept in higher precision.
# ----------------------------------------------------------------------------


def rmsnorm_fp16(h: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    h64 = np.asarray(h, dtype=np.float64)
    r = 1.0 / np.sqrt((h64 * h64).mean(axis=-1, keepdims=True) + eps)
    return (h64 * r).astype(np.float16)


def stack_forward(h0: np.ndarray, layers: list, shape, forced_ids=None) -> dict:
    """Run the residual stack from h0 [T, H]; returns final h (float64) and the
    per-layer x (fp16), ids and w."""
    h = np.asarray(h0, dtype=np.float64).copy()
    xs, ids, ws = [], [], []
    for li, wts in enumerate(layers):
        x = rmsnorm_fp16(h)
        r = moe_layer(x, wts, shape, None if forced_ids is None else forced_ids[li])
        h = h + r["out"]
        xs.append(x)
        ids.append(r["ids"])
        ws.append(r["w"])
    return {"h": h, "x": xs, "ids": ids, "w": ws}


# ----------------------------------------------------------------------------
# Expert-slot pool decisions for partial residency.
#
# [HR] "Partial-residency contract": every routed expert lives in immutable
# host memory; a routed group whose members are all resident reads the GPU
# copies; a miss moves the expert host->device and publishes it only when the
# transfer completes; eviction discards the GPU copy; capacity is fixed before
# admission.  [MS] "What the numbers say": LRU and LFU, with LFU keeping the
# popular experts.  [F51] "Layer 1 - expert persistence cache": per-slot
# frequency counters and last-use timestamps, a slot score of
# frequency*1000 - age, frequencies scaled by 0.75 after every 2*capacity
# misses.
#
# Readings (the pages leave every detail open):
#  * one pool of C slots per routed layer, all free at start;
#  * a per-layer clock ticks once per ensure() call (one routed group);
#  * the group is processed in ascending expert id: first every hit (refresh
#    last-use, counters), then every miss, each taking the lowest free slot,
#    else evicting a resident expert that is not in the group;
#  * victim = minimum key:
#        LRU       (last, id)
#        LFU       (count, last, id), count = calls that touched the expert,
#                  kept across evictions
#        LRU-FREQ  (sfreq*1000 - (clock - last), id), sfreq = 1 on fill,
#                  +1 per hit, float64
#  * LRU-FREQ: after every 2*C misses of the layer, all sfreq *= 0.75.
#
# Next-layer prefetch ([MS] "What the numbers say" and "Method": the next
# layer's experts are guessed by running that layer's router on the current
# state and their copies start while the current layer computes; a guess that
# is used saves its copy, one that is not costs a transfer and a slot, and
# nothing may change the outputs).  Readings:
#  * prefetch(guess) neither ticks the clock nor counts as a use: experts of
#    the guess that are resident are left untouched;
#  * each guessed expert that is not resident (ascending id) is filled like a
#    miss -- lowest free slot, else the minimum-key resident expert outside
#    the guess -- with last = the current clock, its LFU count unchanged,
#    sfreq = 1; it is "pending" until an ensure() names it;
#  * prefetch fills are not misses (they do not advance the LRU-FREQ decay);
#  * an ensure() that names a pending expert counts a hit and marks the first
#    use of the prefetched copy.
# Event codes (the `hit` field): 0 miss, 1 hit, 2 prefetch fill, 3 hit on a
# prefetched copy (its first use), 4 pin fill.
#
# Static / hybrid hot sets ([MS] "What the numbers say": a hot set measured on
# one prompt did worse than LFU on another; [F51] "The simulator": static
# per-layer and global hot sets against dynamic LRU, a static hot+warm sweep).
# Readings:
#  * pin(hot) on a cold pool puts the hot experts, in ascending id, into slots
#    0 .. n-1; they are never victims; the other C - n slots stay dynamic under
#    the policy;
#  * hits on pinned experts are ordinary hits (they refresh last-use and
#    counters like any hit);
#  * a group fits when its experts outside the hot set number at most C - n.
# ----------------------------------------------------------------------------

LRU, LFU, LRU_FREQ = "lru", "lfu", "lru_freq"
EV_MISS, EV_HIT, EV_PREFETCH, EV_PREFETCH_HIT, EV_PIN = 0, 1, 2, 3, 4


@dataclass
class CacheEvent:
    step: int
    layer: int
    expert: int
    hit: int             # EV_MISS, EV_HIT, EV_PREFETCH or EV_PREFETCH_HIT
    slot: int
    victim: int          # evicted expert, -1 if none

    def as_tuple(self):
        return (self.step, self.layer, self.expert, int(self.hit), self.slot, self.victim)


@dataclass
class CacheSim:
    policy: str
    n_experts: int
    capacity: int
    layer: int = 0
    clock: int = 0
    misses: int = 0
    hits: int = 0
    slot_of: dict = field(default_factory=dict)      # expert -> slot
    expert_in: list = field(default_factory=list)    # slot -> expert or -1
    last: dict = field(default_factory=dict)
    count: dict = field(default_factory=dict)
    sfreq: list = field(default_factory=list)
    events: list = field(default_factory=list)
    pending: set = field(default_factory=set)        # prefetched, not yet named by ensure()
    pinned: set = field(default_factory=set)         # hot set: never evicted
    prefetches: int = 0
    prefetch_used: int = 0

    def __post_init__(self):
        assert self.policy in (LRU, LFU, LRU_FREQ)
        self.expert_in = [-1] * self.capacity
        self.sfreq = [0.0] * self.capacity

    def _key(self, e: int):
        if self.policy == LRU:
            return (self.last[e], e)
        if self.policy == LFU:
            return (self.count[e], self.last[e], e)
        s = self.slot_of[e]
        return (self.sfreq[s] * 1000.0 - float(self.clock - self.last[e]), e)

    def ensure(self, group, step: int = 0) -> list:
        """Make every expert of `group` resident; returns its slots in the
        order of `group`.  Appends one CacheEvent per expert."""
        g = sorted(set(int(e) for e in group))
        if len(g) != len(list(group)):
            raise ValueError("group has repeated experts")
        self._check_fits(g)
        self.clock += 1
        in_group = set(g)
        for e in g:
            if e in self.slot_of:
                s = self.slot_of[e]
                self.last[e] = self.clock
                self.count[e] = self.count.get(e, 0) + 1
                self.sfreq[s] += 1.0
                self.hits += 1
                code = EV_HIT
                if e in self.pending:
                    self.pending.discard(e)
                    self.prefetch_used += 1
                    code = EV_PREFETCH_HIT
                self.events.append(CacheEvent(step, self.layer, e, code, s, -1))
        for e in g:
            if e in self.slot_of:
                continue
            victim = -1
            free = [s for s in range(self.capacity) if self.expert_in[s] < 0]
            if free:
                s = free[0]
            else:
                cands = [x for x in self.slot_of if x not in in_group and x not in self.pinned]
                victim = min(cands, key=self._key)
                s = self.slot_of.pop(victim)
                self.pending.discard(victim)
            self.expert_in[s] = e
            self.slot_of[e] = s
            self.last[e] = self.clock
            self.count[e] = self.count.get(e, 0) + 1
            self.sfreq[s] = 1.0
            self.misses += 1
            self.events.append(CacheEvent(step, self.layer, e, EV_MISS, s, victim))
            if self.policy == LRU_FREQ and self.misses % (2 * self.capacity) == 0:
                self.sfreq = [f * 0.75 for f in self.sfreq]
        return [self.slot_of[int(e)] for e in group]

    def _check_fits(self, g):
        outside = [e for e in g if e not in self.pinned]
        if len(outside) > self.capacity - len(self.pinned):
            raise ValueError("group larger than capacity")

    def pin(self, hot, step: int = 0) -> None:
        """Hot set on a cold pool: slots 0 .. n-1 in ascending id, never evicted."""
        h = sorted(set(int(e) for e in hot))
        if len(h) != len(list(hot)):
            raise ValueError("hot set has repeated experts")
        if self.slot_of or self.clock or len(h) >= self.capacity:
            raise ValueError("pin needs a cold pool and at least one dynamic slot")
        for s, e in enumerate(h):
            self.expert_in[s] = e
            self.slot_of[e] = s
            self.last[e] = 0
            self.count[e] = 0
            self.sfreq[s] = 1.0
            self.pinned.add(e)
            self.events.append(CacheEvent(step, self.layer, e, EV_PIN, s, -1))

    def prefetch(self, group, step: int = 0) -> None:
        """Speculative fill of the guessed experts that are not resident (no
        clock tick, no use); appends one EV_PREFETCH event per fill."""
        g = sorted(set(int(e) for e in group))
        if len(g) != len(list(group)):
            raise ValueError("group has repeated experts")
        self._check_fits(g)
        in_group = set(g)
        for e in g:
            if e in self.slot_of:
                continue
            victim = -1
            free = [s for s in range(self.capacity) if self.expert_in[s] < 0]
            if free:
                s = free[0]
            else:
                cands = [x for x in self.slot_of if x not in in_group and x not in self.pinned]
                victim = min(cands, key=self._key)
                s = self.slot_of.pop(victim)
                self.pending.discard(victim)
            self.expert_in[s] = e
            self.slot_of[e] = s
            self.last[e] = self.clock
            self.count[e] = self.count.get(e, 0)
            self.sfreq[s] = 1.0
            self.pending.add(e)
            self.prefetches += 1
            self.events.append(CacheEvent(step, self.layer, e, EV_PREFETCH, s, victim))


# ----------------------------------------------------------------------------
# Offline policy analysis over routing traces ([F51] "The simulator": captured
# router traces are replayed through candidate cache policies offline and the
# hit rate reported per capacity; [MS] "What the numbers say": LRU and LFU hit
# rates at a fixed cache size; [F51] "Layer 1 - expert persistence cache":
# the static top-50% share).  A trace is a list of routed groups (one per
# step) of one layer.
#
# Readings (the pages name the analyses, not their definitions):
#  * OPT is Belady's rule carried over to groups: every expert of the step's
#    group must be resident at once; a miss fills the lowest free slot, else
#    evicts the resident expert outside the group whose next use (first later
#    step naming it) is farthest away, never-used-again counting as infinitely
#    far, ties to the lowest id.  It is pinned against brute force over every
#    eviction choice on tiny traces.
#  * skew: share of all selections that fall on the most-selected ceil(p*E)
#    experts (ties to the lower id) for p = 10%, 20%, 30%; entropy in bits of
#    the selection frequencies; coverage(C) = that share for the top C experts,
#    which is the hit rate a static pin of those C experts would get.
# ----------------------------------------------------------------------------


def opt_hits(groups, capacity: int):
    """(hits, misses) of Belady's farthest-next-use rule over a group trace."""
    gs = [sorted(set(int(e) for e in g)) for g in groups]
    resident = set()
    hits = misses = 0

    def next_use(x, t):
        for u in range(t + 1, len(gs)):
            if x in gs[u]:
                return u
        return math.inf

    for t, g in enumerate(gs):
        if len(g) > capacity:
            raise ValueError("group larger than capacity")
        for e in g:
            if e in resident:
                hits += 1
        for e in g:
            if e in resident:
                continue
            misses += 1
            if len(resident) >= capacity:
                cands = [x for x in resident if x not in g]
                victim = min(cands, key=lambda x: (-next_use(x, t), x))
                resident.remove(victim)
            resident.add(e)
    return hits, misses


def policy_hits(policy: str, groups, n_experts: int, capacity: int, pinned=()):
    """(hits, misses) of one online policy (CacheSim) over a group trace, with
    an optional hot set pinned first."""
    sim = CacheSim(policy, n_experts, capacity)
    if len(pinned):
        sim.pin(pinned)
    for step, g in enumerate(groups):
        sim.ensure(g, step)
    return sim.hits, sim.misses


def selection_counts(groups, n_experts: int) -> np.ndarray:
    c = np.zeros(n_experts, dtype=np.int64)
    for g in groups:
        for e in set(int(x) for x in g):
            c[e] += 1
    return c


def top_share(counts: np.ndarray, n_top: int) -> float:
    """Share of all selections on the n_top most-selected experts (ties to the lower id)."""
    order = sorted(range(len(counts)), key=lambda e: (-int(counts[e]), e))
    total = int(counts.sum())
    return float(sum(int(counts[e]) for e in order[:n_top])) / total if total else 0.0


def skew_report(groups, n_experts: int) -> dict:
    c = selection_counts(groups, n_experts)
    total = int(c.sum())
    ent = 0.0
    for v in c:
        if v:
            p = float(v) / total
            ent -= p * math.log2(p)
    return {"top10": top_share(c, math.ceil(0.1 * n_experts)),
            "top20": top_share(c, math.ceil(0.2 * n_experts)),
            "top30": top_share(c, math.ceil(0.3 * n_experts)),
            "entropy_bits": ent,
            "distinct": int((c > 0).sum())}

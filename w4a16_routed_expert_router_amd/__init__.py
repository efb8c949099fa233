"""MI355X (gfx950) W4A16 routed-expert MoE layer: Python binding.

Thin wrappers over the C ABI in include/moe_w4a16.h (libmoe_w4a16.so).  They
check dtypes/shapes, allocate outputs with PyTorch (device memory and streams
only) and pass pointers; every step of the layer runs in the HIP library.
Importing this package fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import capi
from .capi import (MOE_FLAG_FORCE_GEMV, MOE_FLAG_FORCE_MFMA,  # noqa: F401
                   MOE_FLAG_NO_FUSED, MOE_FLAG_GUESS_AHEAD, MOE_FLAG_ROUTER_EXACT_ALWAYS, MOE_POLICY_LFU, MOE_POLICY_LRU,
                   MOE_POLICY_LRU_FREQ, MOE_RESIDENT_ALL, MoEError)

_lib = capi.load()

POLICIES = {"resident": MOE_RESIDENT_ALL, "lru": MOE_POLICY_LRU, "lfu": MOE_POLICY_LFU,
            "lru_freq": MOE_POLICY_LRU_FREQ}


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, dtype, shape, device, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous {dtype} CUDA tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device.index != device:
        raise ValueError(f"{name} is on cuda:{t.device.index}, context on cuda:{device}")
    return C.c_void_p(t.data_ptr())


def _host(a, dtype, count, name):
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    a = np.ascontiguousarray(a)
    if a.dtype != dtype or a.size != count:
        raise ValueError(f"{name}: expected {count} elements of {dtype}, got {a.size} of {a.dtype}")
    return a


class MoEContext:
    """One library context: `n_layers` MoE layers of one shape on one device."""

    def __init__(self, shape, n_layers=1, max_tokens=64, device=0, policy="resident",
                 slots=0, flags=0, staging_blobs=0, spare_rows=0):
        self.shape = shape
        self.n_layers = n_layers
        self.max_tokens = max_tokens
        self.device = device
        self.policy = POLICIES[policy] if isinstance(policy, str) else int(policy)
        cfg = capi.moe_config(hidden=shape.hidden, n_experts=shape.n_experts, inter=shape.inter,
                              top_k=shape.top_k, renorm=int(shape.renorm), n_layers=n_layers,
                              shared_inter=shape.shared_inter, group=shape.group,
                              max_tokens=max_tokens, device=device, policy=self.policy,
                              slots_per_layer=slots, flags=flags, staging_blobs=staging_blobs,
                              spare_rows=spare_rows)
        h = C.c_void_p()
        self._destroy = _lib.moe_destroy
        capi.check(_lib.moe_create(C.byref(cfg), C.byref(h)), None)
        self._h = h

    # -- lifetime -------------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st):
        capi.check(st, self._h)

    # -- weights --------------------------------------------------------------
    def register_layer(self, layer, w):
        """w: dict with router fp16 [E,H], q uint8 [E,3,I*H/2], s fp16 [E,3,I*H/128]
        (+ shared_q, shared_s), as host numpy arrays or tensors."""
        sh = self.shape
        E, H, I = sh.n_experts, sh.hidden, sh.inter
        router = _host(w["router"], np.float16, E * H, "router")
        q = _host(w["q"], np.uint8, E * 3 * I * H // 2, "q")
        s = _host(w["s"], np.float16, E * 3 * I * H // 128, "s")
        sq = ss = None
        if sh.shared_inter:
            Is = sh.shared_inter
            sq = _host(w["shared_q"], np.uint8, 3 * Is * H // 2, "shared_q")
            ss = _host(w["shared_s"], np.float16, 3 * Is * H // 128, "shared_s")
        self._check(_lib.moe_register_layer(
            self._h, layer, router.ctypes.data, q.ctypes.data, s.ctypes.data,
            None if sq is None else sq.ctypes.data, None if ss is None else ss.ctypes.data))

    # -- hot path -------------------------------------------------------------
    def route(self, layer, x, forced_ids=None, want_logits=False, stream=None):
        sh = self.shape
        T = x.shape[0]
        dev = torch.device("cuda", self.device)
        xp = _dev(x, torch.float16, (T, sh.hidden), self.device, "x")
        fp = None if forced_ids is None else _dev(forced_ids, torch.int32, (T, sh.top_k), self.device, "forced_ids")
        ids = torch.empty((T, sh.top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, sh.top_k), dtype=torch.float32, device=dev)
        logits = torch.empty((T, sh.n_experts), dtype=torch.float32, device=dev) if want_logits else None
        self._check(_lib.moe_route(self._h, layer, xp, T, fp, C.c_void_p(ids.data_ptr()),
                                   C.c_void_p(w.data_ptr()),
                                   None if logits is None else C.c_void_p(logits.data_ptr()),
                                   _stream(stream, self.device)))
        return (ids, w, logits) if want_logits else (ids, w)

    def expert_forward(self, layer, x, ids, w, out=None, stream=None):
        sh = self.shape
        T = x.shape[0]
        xp = _dev(x, torch.float16, (T, sh.hidden), self.device, "x")
        ip = _dev(ids, torch.int32, (T, sh.top_k), self.device, "ids")
        wp = _dev(w, torch.float32, (T, sh.top_k), self.device, "w")
        if out is None:
            out = torch.empty((T, sh.hidden), dtype=torch.float16, device=x.device)
        op = _dev(out, torch.float16, (T, sh.hidden), self.device, "out")
        self._check(_lib.moe_expert_forward(self._h, layer, xp, T, ip, wp, op,
                                            _stream(stream, self.device)))
        return out

    def expert_forward_noalloc(self, layer, x, ids, w, out, stream=None):
        """moe_expert_forward_noalloc: the library's static scratch, no allocation
        in the call; `out` (FP16 [T,H]) must be given."""
        sh = self.shape
        T = x.shape[0]
        xp = _dev(x, torch.float16, (T, sh.hidden), self.device, "x")
        ip = _dev(ids, torch.int32, (T, sh.top_k), self.device, "ids")
        wp = _dev(w, torch.float32, (T, sh.top_k), self.device, "w")
        op = _dev(out, torch.float16, (T, sh.hidden), self.device, "out")
        self._check(_lib.moe_expert_forward_noalloc(self._h, layer, xp, T, ip, wp, op,
                                                    _stream(stream, self.device)))
        return out

    def stack_forward(self, h, layer_begin=0, layer_end=None, forced_ids=None, trace=False,
                      stream=None, h_in=None):
        """h: FP32 [T,H] CUDA tensor, updated in place; with h_in (FP32 [T,H],
        read only) the stack starts from h_in and h receives the result
        (moe_stack_forward_into).  forced_ids: int32 [L,T,k].
        With trace=True returns (x [L,T,H] fp16, ids [L,T,k], w [L,T,k])."""
        sh = self.shape
        T = h.shape[0]
        L = self.n_layers
        layer_end = L if layer_end is None else layer_end
        hp = _dev(h, torch.float32, (T, sh.hidden), self.device, "h")
        fp = None if forced_ids is None else _dev(forced_ids, torch.int32, (L, T, sh.top_k), self.device, "forced_ids")
        xs = ids = ws = None
        if trace:
            xs = torch.zeros((L, T, sh.hidden), dtype=torch.float16, device=h.device)
            ids = torch.full((L, T, sh.top_k), -1, dtype=torch.int32, device=h.device)
            ws = torch.zeros((L, T, sh.top_k), dtype=torch.float32, device=h.device)
        traces = (None if xs is None else C.c_void_p(xs.data_ptr()),
                  None if ids is None else C.c_void_p(ids.data_ptr()),
                  None if ws is None else C.c_void_p(ws.data_ptr()))
        if h_in is None:
            self._check(_lib.moe_stack_forward(self._h, layer_begin, layer_end, hp, T, fp, *traces,
                                               _stream(stream, self.device)))
        else:
            hi = _dev(h_in, torch.float32, (T, sh.hidden), self.device, "h_in")
            self._check(_lib.moe_stack_forward_into(self._h, layer_begin, layer_end, hi, hp, T, fp, *traces,
                                                    _stream(stream, self.device)))
        return (xs, ids, ws) if trace else None

    def check_device_errors(self, stream=None):
        bits = C.c_uint32(0)
        st = _lib.moe_check_device_errors(self._h, _stream(stream, self.device), C.byref(bits))
        if st not in (capi.MOE_OK, capi.MOE_E_DEVICE):
            self._check(st)
        return bits.value

    # -- slot pool --------------------------------------------------------------
    def cache_ensure(self, layer, experts, step=0, stream=None):
        e = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        slots = np.empty_like(e)
        self._check(_lib.moe_cache_ensure(self._h, layer, e.ctypes.data, e.size,
                                          slots.ctypes.data, step, _stream(stream, self.device)))
        return slots

    def cache_prefetch(self, layer, experts, step=0, stream=None):
        e = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        self._check(_lib.moe_cache_prefetch(self._h, layer, e.ctypes.data, e.size, step,
                                            _stream(stream, self.device)))

    def stack_forward_pooled(self, h, step=0, prefetch=True, layer_begin=0, layer_end=None, trace=False,
                             stream=None):
        """Natural routing over the slot pools; h: FP32 [T,H] CUDA tensor, updated in place.
        With trace=True returns (ids [L,T,k], guesses [L,T,k]; -1 where not written)."""
        sh = self.shape
        T = h.shape[0]
        L = self.n_layers
        layer_end = L if layer_end is None else layer_end
        hp = _dev(h, torch.float32, (T, sh.hidden), self.device, "h")
        ids = gs = None
        if trace:
            ids = torch.full((L, T, sh.top_k), -1, dtype=torch.int32, device=h.device)
            gs = torch.full((L, T, sh.top_k), -1, dtype=torch.int32, device=h.device)
        self._check(_lib.moe_stack_forward_pooled(
            self._h, layer_begin, layer_end, hp, T, int(bool(prefetch)), step,
            None if ids is None else C.c_void_p(ids.data_ptr()),
            None if gs is None else C.c_void_p(gs.data_ptr()),
            _stream(stream, self.device)))
        return (ids, gs) if trace else None

    def cache_pin(self, layer, experts, step=0, stream=None):
        e = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        self._check(_lib.moe_cache_pin(self._h, layer, e.ctypes.data, e.size, step,
                                       _stream(stream, self.device)))

    def rmsnorm(self, h, out=None, stream=None):
        sh = self.shape
        T = h.shape[0]
        hp = _dev(h, torch.float32, (T, sh.hidden), self.device, "h")
        if out is None:
            out = torch.empty((T, sh.hidden), dtype=torch.float16, device=h.device)
        op = _dev(out, torch.float16, (T, sh.hidden), self.device, "out")
        self._check(_lib.moe_rmsnorm(self._h, hp, T, op, _stream(stream, self.device)))
        return out

    def cache_stats(self, layer):
        st = capi.moe_cache_counters()
        self._check(_lib.moe_cache_stats(self._h, layer, C.byref(st)))
        return {f: getattr(st, f) for f, _ in capi.moe_cache_counters._fields_}

    def cache_events(self, layer):
        n = C.c_int32(0)
        self._check(_lib.moe_cache_event_log(self._h, layer, None, 0, C.byref(n)))
        cap = 1 << 22
        buf = (capi.moe_cache_event * cap)()
        self._check(_lib.moe_cache_event_log(self._h, layer, buf, cap, C.byref(n)))
        return [buf[i].as_tuple() for i in range(n.value)]

    KERNEL_KINDS = {"logits": 0, "topk": 1, "group": 2, "gateup": 3, "down": 4, "combine": 5,
                    "rmsnorm": 6, "fused": 7, "mfma_gateup": 8, "mfma_down": 9}

    def timer_enable(self, kind):
        self._check(_lib.moe_timer_enable(self._h, -1 if kind is None else self.KERNEL_KINDS[kind]))

    def timer_read(self):
        ms = C.c_double(0.0)
        n = C.c_int64(0)
        self._check(_lib.moe_timer_read(self._h, C.byref(ms), C.byref(n)))
        return ms.value, n.value

    def phase_stamps(self, enable=True):
        """Turn the fused path's phase timestamps on (returns the device buffer,
        [2, grid, stride]: real-time counter, shader-clock counter) or off."""
        g, st, pl = C.c_int32(0), C.c_int32(0), C.c_int32(0)
        self._check(_lib.moe_fused_phase_stamps(self._h, None, 0, C.byref(g), C.byref(st), C.byref(pl)))
        if not enable:
            self._stamps = None
            return None
        buf = torch.zeros((2, g.value, st.value), dtype=torch.int64, device=torch.device("cuda", self.device))
        self._check(_lib.moe_fused_phase_stamps(self._h, C.c_void_p(buf.data_ptr()), buf.numel(),
                                                None, None, None))
        self._stamps = buf            # keeps the buffer alive while the library uses it
        self.stamp_layout = (g.value, st.value, pl.value)
        return buf

    def inject_transfer_failure(self, layer, mode):
        self._check(_lib.moe_debug_inject_transfer_failure(self._h, layer, mode))

    def delay_copies(self, microseconds):
        """Test hook: a bounded wait of `microseconds` on the side stream before
        every host-to-device blob copy (0 turns it off)."""
        self._check(_lib.moe_debug_delay_copies(self._h, microseconds))


class PolicyEngine:
    """Host-only slot-pool decision engine of the library (no GPU needed)."""

    def __init__(self, policy, n_experts, capacity, layer=0):
        p = POLICIES[policy] if isinstance(policy, str) else int(policy)
        self._free = _lib.moe_policy_free
        self._h = _lib.moe_policy_new(p, n_experts, capacity, layer)
        if not self._h:
            raise ValueError("bad policy arguments")

    def access(self, experts, step=0):
        e = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        slots = np.empty_like(e)
        st = _lib.moe_policy_access(self._h, e.ctypes.data, e.size, step, slots.ctypes.data)
        if st != capi.MOE_OK:
            raise MoEError(st, "policy access rejected")
        return slots

    def pin(self, experts, step=0):
        e = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        st = _lib.moe_policy_pin(self._h, e.ctypes.data, e.size, step)
        if st != capi.MOE_OK:
            raise MoEError(st, "policy pin rejected")

    def prefetch(self, experts, step=0):
        e = np.ascontiguousarray(np.asarray(experts, dtype=np.int32))
        st = _lib.moe_policy_prefetch(self._h, e.ctypes.data, e.size, step)
        if st != capi.MOE_OK:
            raise MoEError(st, "policy prefetch rejected")

    def events(self):
        n = _lib.moe_policy_event_count(self._h)
        buf = (capi.moe_cache_event * max(n, 1))()
        m = _lib.moe_policy_events(self._h, buf, n)
        return [buf[i].as_tuple() for i in range(m)]

    def __del__(self):
        if getattr(self, "_h", None):
            self._free(self._h)
            self._h = None


# ---- offline routing-trace analysis (host only) ---------------------------------

def _trace(ids):
    a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    if a.ndim == 1:
        a = a.reshape(-1, 1)
    if a.ndim != 2:
        raise ValueError("a trace is [n_steps, width]")
    return a


def trace_opt(ids, n_experts, capacity):
    """(hits, misses) of Belady's rule for groups over one layer's trace."""
    a = _trace(ids)
    h, m = C.c_int64(), C.c_int64()
    st = _lib.moe_trace_opt(a.ctypes.data, a.shape[0], a.shape[1], n_experts, capacity,
                            C.byref(h), C.byref(m))
    if st != capi.MOE_OK:
        raise MoEError(st, "trace_opt rejected the trace")
    return h.value, m.value


def trace_policy(policy, ids, n_experts, capacity):
    """(hits, misses) of an online slot-pool policy replayed over one layer's trace."""
    a = _trace(ids)
    p = POLICIES[policy] if isinstance(policy, str) else int(policy)
    h, m = C.c_int64(), C.c_int64()
    st = _lib.moe_trace_policy(p, a.ctypes.data, a.shape[0], a.shape[1], n_experts, capacity,
                               C.byref(h), C.byref(m))
    if st != capi.MOE_OK:
        raise MoEError(st, "trace_policy rejected the trace")
    return h.value, m.value


def trace_policy_pinned(policy, ids, n_experts, capacity, hot):
    """(hits, misses) of a policy over one layer's trace with the hot set pinned first."""
    a = _trace(ids)
    p = POLICIES[policy] if isinstance(policy, str) else int(policy)
    hh = np.ascontiguousarray(np.asarray(hot, dtype=np.int32))
    h, m = C.c_int64(), C.c_int64()
    st = _lib.moe_trace_policy_pinned(p, a.ctypes.data, a.shape[0], a.shape[1], n_experts, capacity,
                                      hh.ctypes.data, hh.size, C.byref(h), C.byref(m))
    if st != capi.MOE_OK:
        raise MoEError(st, "trace_policy_pinned rejected the trace")
    return h.value, m.value


def trace_top_share(ids, n_experts, n_top):
    """Share of selections on the n_top most-selected experts (static-pin hit rate)."""
    a = _trace(ids)
    v = C.c_double()
    st = _lib.moe_trace_top_share(a.ctypes.data, a.shape[0], a.shape[1], n_experts, n_top, C.byref(v))
    if st != capi.MOE_OK:
        raise MoEError(st, "trace_top_share rejected the trace")
    return v.value


def trace_skew(ids, n_experts):
    """Top-10/20/30 % shares, entropy (bits), distinct experts and selections of a trace."""
    a = _trace(ids)
    r = capi.moe_skew_report()
    st = _lib.moe_trace_skew(a.ctypes.data, a.shape[0], a.shape[1], n_experts, C.byref(r))
    if st != capi.MOE_OK:
        raise MoEError(st, "trace_skew rejected the trace")
    return {"top10": r.top10, "top20": r.top20, "top30": r.top30, "entropy_bits": r.entropy_bits,
            "distinct": r.distinct, "selections": r.selections}

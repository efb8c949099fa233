"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to a closed form, exact rational
arithmetic, brute force, a hand-decoded value or a hand-worked trace, so
that a plausible slip in the oracle (dropped term, wrong sign, transposed
operand, wrong nibble or scale index, wrong tie-break) fails here.
"""
import itertools
import math
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from fixtures import moe_inputs as fx
from oracle import moe_oracle as ora

# ----------------------------------------------------------------------------
# INT4 layout and dequantisation
# ----------------------------------------------------------------------------


def test_unpack_hand_decoded_bytes():
    # byte 0x21: element 0 = low nibble 1, element 1 = high nibble 2
    packed = np.array([[0x21, 0xF0], [0x8F, 0x07]], dtype=np.uint8)
    assert ora.unpack_int4(packed, 2, 4).tolist() == [[1, 2, 0, 15], [15, 8, 7, 0]]


def test_pack_unpack_roundtrip_all_codes_both_positions():
    codes = torch.tensor([[a, b] for a in range(16) for b in range(16)], dtype=torch.uint8)
    codes = codes.reshape(1, -1)                       # one row, K = 512
    packed = fx.pack_int4(codes).numpy()
    assert np.array_equal(ora.unpack_int4(packed, 1, 512), codes.numpy().astype(np.int64))


def test_dequant_literal():
    # codes [0, 15, 8, 9] with scale 0.5 -> (-8, 7, 0, 1) * 0.5, group 4
    packed = np.array([[0xF0, 0x98]], dtype=np.uint8)
    s = np.array([[0.5]], dtype=np.float16)
    assert ora.dequantize(packed, s, 1, 4, group=4).tolist() == [[-4.0, 3.5, 0.0, 0.5]]


def test_quantisation_error_bound():
    g = torch.Generator().manual_seed(3)
    w = torch.randn(16, 512, generator=g) * 0.02
    w[3, :128] = 0.0                                   # an all-zero group -> s = 0
    codes, s = fx.quantize_int4_g128(w)
    deq = ora.dequantize(fx.pack_int4(codes).numpy(), s.numpy(), 16, 512)
    bound = np.repeat(s.numpy().astype(np.float64), 128, axis=1) / 2
    assert np.all(np.abs(deq - w.double().numpy()) <= bound + 1e-12)
    assert np.all(deq[3, :128] == 0.0)


# ----------------------------------------------------------------------------
# Expert FFN, against pure-Python loops that decode the bytes themselves
# ----------------------------------------------------------------------------

def _py_matrix(packed_row_major, scales, n, k, group):
    """Decode with scalar Python: row r, column c -> nibble of byte r*k/2 + c/2."""
    pb = packed_row_major.reshape(-1).tolist()
    sc = scales.reshape(-1).astype(np.float64).tolist()
    W = [[0.0] * k for _ in range(n)]
    for r in range(n):
        for c in range(k):
            byte = pb[r * (k // 2) + c // 2]
            code = (byte >> (4 * (c % 2))) & 0xF
            W[r][c] = (code - 8) * sc[r * (k // group) + c // group]
    return W


def _py_ffn(xrow, Wg, Wu, Wd):
    I = len(Wg)
    h = []
    for i in range(I):
        gi = sum(a * b for a, b in zip(xrow, Wg[i]))
        ui = sum(a * b for a, b in zip(xrow, Wu[i]))
        h.append(gi / (1.0 + math.exp(-gi)) * ui)
    return [sum(a * b for a, b in zip(h, Wd[n])) for n in range(len(Wd))]


SMALL = fx.MoEShape(hidden=256, n_experts=4, inter=128, top_k=2, renorm=False)


def _small_layer(shape=SMALL, cfg="pin", layer=0):
    w = fx.layer_weights(shape, cfg, layer, device="cpu")
    return {k: v.numpy() for k, v in w.items()}


def test_expert_ffn_against_python_loops():
    wts = _small_layer()
    H, I = SMALL.hidden, SMALL.inter
    x = fx.activations(("pin-ffn",), 2, H).numpy()
    e = 2
    mats = ora.expert_matrices(wts["q"][e], wts["s"][e], H, I)
    got = ora.expert_ffn(x.astype(np.float64), *mats)
    Wg = _py_matrix(wts["q"][e][0], wts["s"][e][0], I, H, 128)
    Wu = _py_matrix(wts["q"][e][1], wts["s"][e][1], I, H, 128)
    Wd = _py_matrix(wts["q"][e][2], wts["s"][e][2], H, I, 128)
    for t in range(2):
        ref = _py_ffn([float(v) for v in x[t]], Wg, Wu, Wd)
        np.testing.assert_allclose(got[t], ref, rtol=1e-9, atol=1e-12)


def test_moe_layer_against_python_loops():
    wts = _small_layer()
    H, I, k = SMALL.hidden, SMALL.inter, SMALL.top_k
    T = 3
    x = fx.activations(("pin-layer",), T, H).numpy()
    res = ora.moe_layer(x, wts, SMALL)
    # routing from Fraction-exact logits and brute-force ordering
    for t in range(T):
        logits = [_fraction_dot(x[t], wts["router"][e]) for e in range(SMALL.n_experts)]
        order = sorted(range(SMALL.n_experts), key=lambda e: (-logits[e], e))
        assert res["ids"][t].tolist() == order[:k]
        m = max(float(v) for v in logits)
        p = [math.exp(float(v) - m) for v in logits]
        ssum = sum(p)
        out = [0.0] * H
        for j, e in enumerate(order[:k]):
            wj = p[e] / ssum
            assert abs(wj - res["w"][t, j]) < 1e-6 * wj
            mats = [_py_matrix(wts["q"][e][m_], wts["s"][e][m_], *nk, 128)
                    for m_, nk in ((0, (I, H)), (1, (I, H)), (2, (H, I)))]
            y = _py_ffn([float(v) for v in x[t]], *mats)
            out = [o + wj * yy for o, yy in zip(out, y)]
        np.testing.assert_allclose(res["out"][t], out, rtol=1e-6, atol=1e-9)


def test_identical_experts_scale_by_weight_sum():
    wts = _small_layer()
    for key in ("q", "s"):
        wts[key] = np.repeat(wts[key][:1], SMALL.n_experts, axis=0)
    x = fx.activations(("pin-ident",), 4, SMALL.hidden).numpy()
    res = ora.moe_layer(x, wts, SMALL)
    mats = ora.expert_matrices(wts["q"][0], wts["s"][0], SMALL.hidden, SMALL.inter)
    dense = ora.expert_ffn(x.astype(np.float64), *mats)
    np.testing.assert_allclose(res["out"], res["w"].sum(1, keepdims=True) * dense, rtol=1e-12, atol=1e-12)


def test_k1_renorm_is_dense_ffn_and_shared_expert_adds():
    shape = fx.MoEShape(hidden=256, n_experts=4, inter=128, top_k=1, renorm=True, shared_inter=128)
    wts = _small_layer(shape, cfg="pin-k1")
    x = fx.activations(("pin-k1",), 3, shape.hidden).numpy()
    res = ora.moe_layer(x, wts, shape)
    assert np.all(res["w"] == 1.0)
    H, I = shape.hidden, shape.inter
    for t in range(3):
        e = res["ids"][t, 0]
        routed = ora.expert_ffn(x[t:t + 1].astype(np.float64), *ora.expert_matrices(wts["q"][e], wts["s"][e], H, I))
        shared = _py_ffn([float(v) for v in x[t]],
                         _py_matrix(wts["shared_q"][0], wts["shared_s"][0], I, H, 128),
                         _py_matrix(wts["shared_q"][1], wts["shared_s"][1], I, H, 128),
                         _py_matrix(wts["shared_q"][2], wts["shared_s"][2], H, I, 128))
        np.testing.assert_allclose(res["out"][t], routed[0] + np.array(shared), rtol=1e-9, atol=1e-12)


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0])
    s = ora.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(s[1] - 0.7310585786300049) < 1e-15
    assert abs(s[2] - (-1.0 / (1.0 + math.e))) < 1e-15
    assert abs(s[3] - 40.0) < 1e-12 and abs(s[4]) < 1e-15


# ----------------------------------------------------------------------------
# Exact router logits
# ----------------------------------------------------------------------------

def _fraction_dot(x, w):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, w))


def _fraction_to_f32(F):
    """Nearest FP32 to the rational F, ties to even (independent of the oracle)."""
    c = np.float32(float(F))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = None
    for v in cands:
        d = abs(Fraction(float(v)) - F)
        even = (int(np.array(v, dtype=np.float32).view(np.uint32)) & 1) == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, v)
    return np.float32(best[1])


def _random_fp16(rng, n, wide):
    if wide:   # random finite bit patterns: subnormals, tiny and huge values
        bits = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
        v = bits.view(np.float16)
        return np.where(np.isfinite(v), v, np.float16(1.0)).astype(np.float16)
    return rng.standard_normal(n).astype(np.float16)


@pytest.mark.parametrize("wide", [False, True])
def test_router_logits_equal_fraction_rounding(wide):
    rng = np.random.default_rng(11 + wide)
    T, E, H = 3, 5, 40
    x = _random_fp16(rng, T * H, wide).reshape(T, H)
    wr = _random_fp16(rng, E * H, wide).reshape(E, H)
    got = ora.router_logits(x, wr)
    for t in range(T):
        for e in range(E):
            want = _fraction_to_f32(_fraction_dot(x[t], wr[e]))
            assert got[t, e].view(np.uint32) == want.view(np.uint32), (t, e)


def test_exact_dot_matches_python_object_matmul():
    rng = np.random.default_rng(5)
    x = _random_fp16(rng, 4 * 2048, True).reshape(4, 2048)
    w = _random_fp16(rng, 6 * 2048, True).reshape(6, 2048)
    xi, wi = ora.fp16_as_int(x), ora.fp16_as_int(w)
    want = np.dot(xi.astype(object), wi.T.astype(object))
    assert (ora.exact_dot_ints(xi, wi) == want).all()


def test_fp16_as_int_literal():
    v = np.array([1.0, -2.0 ** -24, 65504.0, 0.5], dtype=np.float16)
    assert ora.fp16_as_int(v).tolist() == [1 << 24, -1, 65504 << 24, 1 << 23]


def test_rounding_midpoints_ties_to_even():
    # 1 + 2^-24 is halfway between 1 and 1 + 2^-23: ties to even -> 1
    x = np.array([[1.0, 2.0 ** -12]], dtype=np.float16)
    assert ora.router_logits(x, x)[0, 0] == np.float32(1.0)
    # 1 + 3*2^-24 is halfway between 1+2^-23 (odd) and 1+2^-22 (even) -> 1+2^-22
    x3 = np.array([[1.0, 2.0 ** -12, 2.0 ** -12, 2.0 ** -12]], dtype=np.float16)
    assert ora.router_logits(x3, x3)[0, 0] == np.float32(1.0 + 2.0 ** -22)
    # just above the first midpoint rounds up
    xa = np.array([[1.0, 2.0 ** -12, 2.0 ** -24]], dtype=np.float16)
    wa = np.array([[1.0, 2.0 ** -12, 1.0]], dtype=np.float16)
    assert ora.router_logits(xa, wa)[0, 0] == np.float32(1.0 + 2.0 ** -23)


def test_round_matches_numpy_when_double_is_exact():
    rnd = random.Random(7)
    for _ in range(3000):
        S = rnd.randrange(-(1 << 52), 1 << 52) >> rnd.randrange(0, 50)
        want = np.float32(S * 2.0 ** -48)            # S*2^-48 exact in double: one rounding
        assert ora.round_int_scaled_to_f32(S, -48).view(np.uint32) == want.view(np.uint32)


def test_duplicate_router_rows_pick_lowest_id():
    rng = np.random.default_rng(2)
    wr = rng.standard_normal((6, 64)).astype(np.float16)
    wr[4] = wr[1]
    x = np.sign(wr[1:2].astype(np.float32)).astype(np.float16)  # x . wr[1] is the maximum
    logits = ora.router_logits(x, wr)
    assert logits[0, 1] == logits[0, 4]
    ids = ora.topk(logits, 2)
    assert ids[0].tolist() == [1, 4]


# ----------------------------------------------------------------------------
# Top-k, softmax, combine weights
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("E,k", [(5, 2), (7, 3), (10, 4), (6, 1)])
def test_topk_brute_force_subsets(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for _ in range(30):
        # few distinct values -> many ties
        logits = rng.integers(-2, 3, size=(1, E)).astype(np.float32) * np.float32(0.25)
        ids = ora.topk(logits, k)[0].tolist()

        def beats(a, b):       # a ranks before b
            return logits[0, a] > logits[0, b] or (logits[0, a] == logits[0, b] and a < b)

        valid = [S for S in itertools.combinations(range(E), k)
                 if all(beats(a, b) for a in S for b in range(E) if b not in S)]
        assert len(valid) == 1
        assert sorted(ids) == list(valid[0])
        assert all(beats(ids[i], ids[i + 1]) for i in range(k - 1))


def test_softmax_two_expert_closed_form_and_sum():
    lg = np.array([[0.5, -1.25]], dtype=np.float32)
    p = ora.softmax(lg)
    assert abs(p[0, 0] - 1.0 / (1.0 + math.exp(-1.75))) < 1e-15
    rng = np.random.default_rng(0)
    big = rng.standard_normal((8, 512)).astype(np.float32)
    assert np.allclose(ora.softmax(big).sum(1), 1.0, atol=1e-13)
    assert np.allclose(ora.softmax(big + np.float32(3.0)), ora.softmax(big), atol=1e-13)


def test_combine_weights_are_gathered_probabilities():
    rng = np.random.default_rng(1)
    lg = rng.standard_normal((5, 64)).astype(np.float32)
    p = ora.softmax(lg)
    ids = ora.topk(lg, 8)
    w = ora.combine_weights(p, ids, renorm=False)
    for t in range(5):
        for j in range(8):
            assert w[t, j] == p[t, ids[t, j]]
    wr = ora.combine_weights(p, ids, renorm=True)
    assert np.allclose(wr.sum(1), 1.0, atol=1e-15)
    assert np.allclose(wr * w.sum(1, keepdims=True), w, rtol=1e-14)


# ----------------------------------------------------------------------------
# Stack glue
# ----------------------------------------------------------------------------

def test_rmsnorm_constant_vector_closed_form():
    h = np.full((2, 256), 3.0)
    x = ora.rmsnorm_fp16(h)
    assert np.all(x == np.float16(3.0 / math.sqrt(9.0 + 1e-5)))


def _fp16_of_exact(num: Fraction, den_sq: Fraction) -> np.float16:
    """FP16 nearest to num / sqrt(den_sq), from 60-digit decimal arithmetic;
    the value is checked to lie far from an FP16 rounding midpoint, so the
    rounding through float64 cannot differ from rounding the exact value."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    v = Decimal(num.numerator) / Decimal(num.denominator) / (
        Decimal(den_sq.numerator) / Decimal(den_sq.denominator)).sqrt()
    r = np.float16(float(v))
    lo, hi = np.nextafter(r, np.float16(-np.inf)), np.nextafter(r, np.float16(np.inf))
    for nb in (lo, hi):
        mid = (Decimal(float(r)) + Decimal(float(nb))) / 2
        assert abs(v - mid) > abs(Decimal(float(nb)) - Decimal(float(r))) / 64
    return r


def test_rmsnorm_alternating_vector_exact():
    """h = [3, 4, 3, 4, ...]: mean(h^2) = 12.5 (mean(h)^2 would be 12.25, and
    a sum instead of a mean 3200), so x = h / sqrt(12.5 + 1e-5) in exact
    arithmetic, rounded once to FP16."""
    H = 256
    h = np.tile(np.array([3.0, 4.0]), H // 2)[None, :]
    x = ora.rmsnorm_fp16(h)
    ms = Fraction(25, 2) + Fraction(1, 100000)
    want3, want4 = _fp16_of_exact(Fraction(3), ms), _fp16_of_exact(Fraction(4), ms)
    assert np.all(x[0, 0::2] == want3) and np.all(x[0, 1::2] == want4)
    # the readings this pin rejects give other FP16 values
    assert want3 != np.float16(3.0 / 3.5) and want4 != np.float16(4.0 / 3.5)


def test_rmsnorm_small_norm_pins_eps():
    """|h_i| = 2^-10 for every i: mean(h^2) = 2^-20 ~ 9.5e-7, the same order as
    eps, so eps = 1e-5 decides the result: x = 2^-10 / sqrt(2^-20 + 1e-5)
    (~0.3028), where eps = 0 gives 1, eps = 1e-6 gives ~0.70 and eps = 1e-4
    gives ~0.0976."""
    H = 512
    sgn = np.where(np.arange(H) % 3 == 0, -1.0, 1.0)
    h = (sgn * 2.0 ** -10)[None, :]
    x = ora.rmsnorm_fp16(h)
    ms = Fraction(1, 2 ** 20) + Fraction(1, 100000)
    want = _fp16_of_exact(Fraction(1, 2 ** 10), ms)
    assert np.all(x[0] == (sgn * float(want)).astype(np.float16))
    for eps in (0.0, 1e-6, 1e-4):
        other = _fp16_of_exact(Fraction(1, 2 ** 10), Fraction(1, 2 ** 20) + Fraction(eps))
        assert other != want


def test_rmsnorm_rows_are_independent():
    """Each token (row) is normalised by its own mean square."""
    h = np.stack([np.full(256, 3.0), np.tile([3.0, 4.0], 128)])
    x = ora.rmsnorm_fp16(h)
    assert np.all(x[0] == np.float16(3.0 / math.sqrt(9.0 + 1e-5)))
    assert np.array_equal(x[1], ora.rmsnorm_fp16(h[1:2])[0])


def _py_rmsnorm_fp16(hrow):
    ms = sum(v * v for v in hrow) / len(hrow)
    r = 1.0 / math.sqrt(ms + 1e-5)
    return [float(np.float16(v * r)) for v in hrow]


def _py_layer(xrow, wts, shape):
    """One token through one layer with scalar Python: Fraction-exact logits,
    (logit desc, id asc) order, softmax probabilities, rank-ordered sum."""
    H, I, k = shape.hidden, shape.inter, shape.top_k
    logits = [_fraction_dot(np.asarray(xrow, dtype=np.float16), wts["router"][e])
              for e in range(shape.n_experts)]
    order = sorted(range(shape.n_experts), key=lambda e: (-logits[e], e))[:k]
    m = max(float(v) for v in logits)
    p = [math.exp(float(v) - m) for v in logits]
    tot = sum(p)
    out = [0.0] * H
    for e in order:
        mats = [_py_matrix(wts["q"][e][m_], wts["s"][e][m_], *nk, 128)
                for m_, nk in ((0, (I, H)), (1, (I, H)), (2, (H, I)))]
        y = _py_ffn(xrow, *mats)
        out = [o + p[e] / tot * yy for o, yy in zip(out, y)]
    return out, order


def test_stack_two_layer_recurrence_python_loops():
    """Two layers, one token: h1 = h0 + L0(n(h0)), h2 = h1 + L1(n(h1)), with
    n, the routing and the FFN written as scalar Python loops.  Normalising h0
    at both layers, skipping the residual, or reusing layer 0's weights would
    each give another h2 (checked below, so the pin keeps its power)."""
    sh = SMALL
    l0, l1 = _small_layer(layer=0), _small_layer(layer=1)
    h0 = fx.activations(("pin-stack-2",), 1, sh.hidden).numpy()
    res = ora.stack_forward(h0, [l0, l1], sh)
    h = [float(v) for v in h0[0]]
    x0 = _py_rmsnorm_fp16(h)
    o0, ids0 = _py_layer(x0, l0, sh)
    h1 = [a + b for a, b in zip(h, o0)]
    x1 = _py_rmsnorm_fp16(h1)
    o1, ids1 = _py_layer(x1, l1, sh)
    h2 = [a + b for a, b in zip(h1, o1)]
    assert res["ids"][0][0].tolist() == ids0 and res["ids"][1][0].tolist() == ids1
    assert np.array_equal(res["x"][1][0].astype(np.float64), np.array(x1))
    np.testing.assert_allclose(res["h"][0], h2, rtol=1e-9, atol=1e-9)
    # slips this pin must catch
    stale, _ = _py_layer(x0, l1, sh)
    wrong_norm = [a + b for a, b in zip(h1, stale)]
    same_w, _ = _py_layer(x1, l0, sh)
    wrong_layer = [a + b for a, b in zip(h1, same_w)]
    no_resid = o1
    for bad in (wrong_norm, wrong_layer, no_resid):   # each far outside the 1e-9 tolerance above
        assert np.max(np.abs(np.array(bad) - np.array(h2))) > 1e-6


def test_stack_zero_weights_is_identity_and_one_layer_is_layer():
    wts = _small_layer()
    zero = dict(wts)
    zero["q"] = np.full_like(wts["q"], 0x88)          # every code 8 -> weight 0
    h0 = fx.activations(("pin-stack",), 2, SMALL.hidden).numpy()
    res = ora.stack_forward(h0, [zero, zero], SMALL)
    assert np.array_equal(res["h"], h0.astype(np.float64))
    one = ora.stack_forward(h0, [wts], SMALL)
    lay = ora.moe_layer(ora.rmsnorm_fp16(h0), wts, SMALL)
    assert np.array_equal(one["h"], h0.astype(np.float64) + lay["out"])


# ----------------------------------------------------------------------------
# Cache decisions: hand-worked traces
# ----------------------------------------------------------------------------

def _run(policy, C, groups, E=16):
    sim = ora.CacheSim(policy, E, C)
    for step, g in enumerate(groups):
        sim.ensure(g, step)
    return [(e.expert, int(e.hit), e.slot, e.victim) for e in sim.events]


TRACE = [[1], [2], [1], [3], [2], [1]]


def test_lru_hand_trace():
    assert _run(ora.LRU, 2, TRACE) == [
        (1, 0, 0, -1), (2, 0, 1, -1), (1, 1, 0, -1), (3, 0, 1, 2), (2, 0, 0, 1), (1, 0, 1, 3)]


def test_lfu_hand_trace():
    assert _run(ora.LFU, 2, TRACE) == [
        (1, 0, 0, -1), (2, 0, 1, -1), (1, 1, 0, -1), (3, 0, 1, 2), (2, 0, 1, 3), (1, 1, 0, -1)]
    # LFU keeps a frequent expert that LRU drops
    assert _run(ora.LFU, 2, [[1], [1], [2], [3], [1]])[-1] == (1, 1, 0, -1)
    assert _run(ora.LRU, 2, [[1], [1], [2], [3], [1]])[-1][1] == 0


def test_lru_freq_hand_trace_with_decay():
    ev = _run(ora.LRU_FREQ, 2, TRACE + [[4]])
    assert ev == [(1, 0, 0, -1), (2, 0, 1, -1), (1, 1, 0, -1), (3, 0, 1, 2), (2, 0, 1, 3),
                  (1, 1, 0, -1), (4, 0, 1, 2)]
    sim = ora.CacheSim(ora.LRU_FREQ, 16, 2)
    for g in TRACE + [[4]]:
        sim.ensure(g)
    # fills: 1->1, 2->1, hit 1->2; 4th miss decays [2,1] -> [1.5, 0.75]; hit -> 2.5; refill -> 1
    assert sim.sfreq == [2.5, 1.0]
    # frequency protects an older expert: LRU-FREQ evicts 2, LRU evicts 1
    assert _run(ora.LRU_FREQ, 2, [[1], [1], [1], [2], [3]])[-1] == (3, 0, 1, 2)
    assert _run(ora.LRU, 2, [[1], [1], [1], [2], [3]])[-1] == (3, 0, 0, 1)


def test_multi_expert_groups_hits_first_then_misses():
    ev = _run(ora.LRU, 3, [[5, 1], [1, 7], [2, 5]])
    assert ev == [(1, 0, 0, -1), (5, 0, 1, -1), (1, 1, 0, -1), (7, 0, 2, -1),
                  (5, 1, 1, -1), (2, 0, 0, 1)]


def test_cyclic_walk_lru_zero_hits():
    C = 8
    walk = [[e] for e in list(range(C + 1)) * 6]
    ev = _run(ora.LRU, C, walk, E=C + 1)
    assert sum(h for _, h, _, _ in ev) == 0


@pytest.mark.parametrize("policy", [ora.LRU, ora.LFU, ora.LRU_FREQ])
def test_working_set_within_capacity_misses_once(policy):
    rng = np.random.default_rng(9)
    ws = rng.choice(64, size=12, replace=False)
    groups = [sorted(rng.choice(ws, size=4, replace=False).tolist()) for _ in range(50)]
    ev = _run(policy, 12, groups, E=64)
    assert sum(1 - h for _, h, _, _ in ev) == len(set(np.concatenate(groups).tolist()))


def _belady_hits(seq, C):
    res, hits = set(), 0
    for i, e in enumerate(seq):
        if e in res:
            hits += 1
            continue
        if len(res) >= C:
            def nxt(x):
                for j in range(i + 1, len(seq)):
                    if seq[j] == x:
                        return j
                return 1 << 30
            res.remove(max(res, key=nxt))
        res.add(e)
    return hits


@pytest.mark.parametrize("policy", [ora.LRU, ora.LFU, ora.LRU_FREQ])
def test_hits_never_exceed_belady_on_k1_traces(policy):
    tr = fx.zipf_trace("pin-belady", 400, 1, 32, 1)
    seq = tr[:, 0, 0].tolist()
    for C in (2, 4, 8):
        ev = _run(policy, C, [[e] for e in seq], E=32)
        assert sum(h for _, h, _, _ in ev) <= _belady_hits(seq, C)


def test_group_larger_than_capacity_rejected():
    sim = ora.CacheSim(ora.LRU, 16, 2)
    with pytest.raises(ValueError):
        sim.ensure([1, 2, 3])


# ---------------------------------------------------------------------------
# Offline policy analysis: OPT bound and router skew
# ---------------------------------------------------------------------------

def _brute_max_hits(groups, C):
    """Largest hit count over every eviction choice (free slots always used first)."""
    from functools import lru_cache
    gs = [tuple(sorted(set(g))) for g in groups]

    @lru_cache(maxsize=None)
    def go(t, res):
        if t == len(gs):
            return 0
        g = gs[t]
        hits = sum(1 for e in g if e in res)
        missing = [e for e in g if e not in res]

        def place(i, cur):
            if i == len(missing):
                return go(t + 1, cur)
            e = missing[i]
            if len(cur) < C:
                return place(i + 1, cur | frozenset([e]))
            best = -1
            for v in cur:
                if v not in g:
                    best = max(best, place(i + 1, (cur - frozenset([v])) | frozenset([e])))
            return best

        return hits + place(0, res)

    return go(0, frozenset())


@pytest.mark.parametrize("seed", range(6))
def test_opt_equals_brute_force_on_tiny_traces(seed):
    rng = np.random.default_rng(100 + seed)
    E, C, steps = 6, 2 + seed % 2, 9
    groups = [rng.choice(E, size=int(rng.integers(1, C + 1)), replace=False).tolist() for _ in range(steps)]
    h, m = ora.opt_hits(groups, C)
    assert h == _brute_max_hits(groups, C)
    assert h + m == sum(len(g) for g in groups)


@pytest.mark.parametrize("C", [16, 32, 48])
def test_online_policies_never_beat_opt_on_group_traces(C):
    tr = fx.zipf_trace("pin-opt", 200, 1, 64, 8)
    groups = [tr[s, 0].tolist() for s in range(tr.shape[0])]
    oh, om = ora.opt_hits(groups, C)
    for policy in (ora.LRU, ora.LFU, ora.LRU_FREQ):
        h, m = ora.policy_hits(policy, groups, 64, C)
        assert h <= oh and h + m == oh + om


def test_opt_working_set_within_capacity_misses_once():
    rng = np.random.default_rng(5)
    ws = rng.choice(64, size=10, replace=False)
    groups = [rng.choice(ws, size=4, replace=False).tolist() for _ in range(40)]
    _, m = ora.opt_hits(groups, 10)
    assert m == len(set(np.concatenate(groups).tolist()))


def test_skew_closed_forms():
    E = 20
    uniform = [[e] for e in range(E)] * 3          # every expert equally often
    r = ora.skew_report(uniform, E)
    assert r["entropy_bits"] == pytest.approx(np.log2(E), abs=1e-12)
    assert r["top10"] == pytest.approx(2 / E) and r["top30"] == pytest.approx(6 / E)
    assert r["distinct"] == E
    single = [[7]] * 5
    r = ora.skew_report(single, E)
    assert r["entropy_bits"] == 0.0 and r["top10"] == 1.0 and r["distinct"] == 1
    # counts 3, 1 over E = 10: top-10% (1 expert) = 3/4, entropy of (3/4, 1/4)
    r = ora.skew_report([[2], [2], [2], [5]], 10)
    assert r["top10"] == pytest.approx(0.75)
    assert r["entropy_bits"] == pytest.approx(-(0.75 * np.log2(0.75) + 0.25 * np.log2(0.25)), abs=1e-12)
    # a tie for the top place goes to the lower id
    c = np.array([0, 4, 0, 4, 1])
    assert ora.top_share(c, 1) == pytest.approx(4 / 9)


# ---- next-layer prefetch in the slot-pool simulator (hand-worked traces) ----------

def _ev(sim):
    return [(e.step, e.expert, int(e.hit), e.slot, e.victim) for e in sim.events]


def test_prefetch_lru_hand_worked_trace():
    # C=3, LRU.  step 0 fills 1, 2; a guess {2, 5} fills only 5 (2 is resident,
    # untouched); step 1 uses 5 (first use of a prefetched copy) and misses 3,
    # evicting 1 (last 1, lower id than 2); a guess {4} evicts 2 (last 1);
    # step 2 hits 3 and misses 2, evicting the unused prefetched 4 (last 1)
    # rather than 5 (last 2).
    sim = ora.CacheSim(ora.LRU, 8, 3)
    sim.ensure([1, 2], step=0)
    sim.prefetch([2, 5], step=1)
    sim.ensure([3, 5], step=1)
    sim.prefetch([4], step=2)
    sim.ensure([2, 3], step=2)
    M, H, PF, PH = ora.EV_MISS, ora.EV_HIT, ora.EV_PREFETCH, ora.EV_PREFETCH_HIT
    assert _ev(sim) == [(0, 1, M, 0, -1), (0, 2, M, 1, -1), (1, 5, PF, 2, -1), (1, 5, PH, 2, -1),
                        (1, 3, M, 0, 1), (2, 4, PF, 1, 2), (2, 3, H, 0, -1), (2, 2, M, 1, 4)]
    assert (sim.hits, sim.misses, sim.prefetches, sim.prefetch_used) == (2, 4, 2, 1)
    assert sim.pending == set()


def test_prefetch_is_not_a_use_for_lfu():
    # 1 was used once; 3 is prefetched and never used: its count stays 0, so the
    # next miss evicts 3, not 1 (had the prefetch counted, keys would tie on
    # (count 1, last 1) and the lower id 1 would go)
    sim = ora.CacheSim(ora.LFU, 8, 2)
    sim.ensure([1], step=0)
    sim.prefetch([3], step=1)
    sim.ensure([4], step=1)
    assert _ev(sim)[-1] == (1, 4, ora.EV_MISS, 1, 3)


def test_prefetch_fills_do_not_advance_lru_freq_decay():
    # C=2: the decay comes after every 4 misses.  A prefetch of 0, then misses
    # 1, 2, 3, 4 (hit on 0 in between): the decay runs right after the 4th
    # miss, so sfreq = [2 * 0.75, 1 * 0.75]; counting the prefetch as a miss
    # would have decayed after miss 3 and left [1.5, 1.0].
    sim = ora.CacheSim(ora.LRU_FREQ, 8, 2)
    sim.prefetch([0], step=0)
    sim.ensure([1], step=0)
    sim.ensure([0], step=1)
    sim.ensure([2], step=2)
    sim.ensure([3], step=3)
    sim.ensure([4], step=4)
    assert [e.victim for e in sim.events if e.hit == ora.EV_MISS] == [-1, 1, 2, 3]
    assert sim.sfreq == [1.5, 0.75]
    assert sim.misses == 4 and sim.prefetches == 1 and sim.prefetch_used == 1


@pytest.mark.parametrize("policy", [ora.LRU, ora.LFU, ora.LRU_FREQ])
def test_prefetch_of_the_exact_next_group_leaves_no_demand_miss(policy):
    # after prefetch(G) every expert of G is resident (a fill never evicts a
    # member of the guess), so ensure(G) right after it has no miss and uses
    # every prefetched copy
    trace = fx.zipf_trace("pin-prefetch", 60, 1, 32, 6)[:, 0, :]
    sim = ora.CacheSim(policy, 32, 8)
    sim.ensure(trace[0], step=0)
    first = sim.misses
    for t in range(1, len(trace)):
        sim.prefetch(trace[t], step=t)
        sim.ensure(trace[t], step=t)
    assert sim.misses == first
    assert sim.prefetch_used == sim.prefetches


@pytest.mark.parametrize("policy", [ora.LRU, ora.LFU, ora.LRU_FREQ])
def test_empty_prefetch_changes_nothing(policy):
    trace = fx.zipf_trace("pin-prefetch-empty", 40, 1, 24, 5)[:, 0, :]
    a, b = ora.CacheSim(policy, 24, 7), ora.CacheSim(policy, 24, 7)
    for t, g in enumerate(trace):
        a.ensure(g, step=t)
        b.prefetch([], step=t)
        b.ensure(g, step=t)
    assert _ev(a) == _ev(b)


# ---- static / hybrid hot sets in the slot-pool simulator -------------------------

def test_pinned_expert_is_never_the_victim_lru():
    # C=3 with expert 6 pinned in slot 0 (last-use 0, so LRU would drop it
    # first were it not pinned): the miss of 3 evicts 1 instead (last 1,
    # lower id than 2); a hit on 6 is an ordinary hit
    sim = ora.CacheSim(ora.LRU, 8, 3)
    sim.pin([6], step=0)
    sim.ensure([1, 2], step=0)
    sim.ensure([3], step=1)
    sim.ensure([4, 6], step=2)
    M, H, P = ora.EV_MISS, ora.EV_HIT, ora.EV_PIN
    assert _ev(sim) == [(0, 6, P, 0, -1), (0, 1, M, 1, -1), (0, 2, M, 2, -1), (1, 3, M, 1, 1),
                        (2, 6, H, 0, -1), (2, 4, M, 2, 2)]
    assert (sim.hits, sim.misses) == (1, 4)


def test_pinned_capacity_rules():
    sim = ora.CacheSim(ora.LFU, 8, 3)
    sim.pin([6, 7])
    sim.ensure([1, 6, 7])              # one expert outside the hot set: fits one dynamic slot
    with pytest.raises(ValueError):
        sim.ensure([1, 2])             # two outside, one dynamic slot
    with pytest.raises(ValueError):
        ora.CacheSim(ora.LRU, 8, 3).pin([0, 1, 2])   # no dynamic slot left
    warm = ora.CacheSim(ora.LRU, 8, 3)
    warm.ensure([1])
    with pytest.raises(ValueError):
        warm.pin([2])                  # not a cold pool


@pytest.mark.parametrize("policy", [ora.LRU, ora.LFU, ora.LRU_FREQ])
def test_pinned_hot_set_always_hits(policy):
    # every selection of a pinned expert is a hit, so hits >= those selections;
    # pins are not misses
    trace = fx.zipf_trace("pin-hot", 80, 1, 32, 6)[:, 0, :]
    groups = [sorted(int(e) for e in g) for g in trace]
    counts = ora.selection_counts(groups, 32)
    hot = sorted(range(32), key=lambda e: (-int(counts[e]), e))[:8]
    hits, misses = ora.policy_hits(policy, groups, 32, 14, pinned=hot)
    assert hits >= int(sum(counts[e] for e in hot))
    assert hits + misses == sum(len(g) for g in groups)

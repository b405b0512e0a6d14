"""Pins of the oracle's elementary pieces against the mathematics and against
independent library routines (numpy's binary16, Python's decimal, scipy).

Section tags refer to the page "Runtime-Certified Bounded-Error Quantized
Attention" (technical summary): [Meth-1] tiered storage, [Meth-2] two-term
error decomposition, [Meth-3] adaptive precision and fallback ladder.
"""
import itertools
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import datagen
import oracle

getcontext().prec = 60


def f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def h2f(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


# -- binary16 -----------------------------------------------------------------

def test_h2f_matches_numpy_on_every_pattern():
    L = oracle.lib()
    pats = np.arange(65536, dtype=np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([L.orc_h2f(int(p)) for p in pats], np.float32)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.isinf(got[np.isinf(ref)]))
    assert np.all(np.isnan(got[np.isnan(ref)]))


def test_f2h_up_is_the_smallest_half_above():
    L = oracle.lib()
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.uniform(0, 1, 3000), rng.uniform(0, 60000, 3000),
                         10.0 ** rng.uniform(-9, -3, 3000)]).astype(np.float32)
    xs = np.concatenate([xs, h2f(np.arange(1, 0x7C00, 97)).astype(np.float32)])
    for x in xs:
        h = L.orc_f2h_up(float(x))
        assert h2f(h) >= x
        assert h == 0 or h2f(h - 1) < x


def test_datagen_f16_rounding_matches_numpy():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-8, 4.6, 20000),
                        [0.0, -0.0, 65504.0, 65519.9, 6e-8, 3e-8, 2.9e-8]])
    assert np.array_equal(datagen.to_f16(x), x.astype(np.float16).view(np.uint16))


def test_philox_known_answer():
    # Philox4x32-10, zero counter and key (Salmon et al., SC'11 test vectors)
    assert [hex(v) for v in datagen.philox([0, 0, 0, 0], [0, 0])] == \
        ["0x6627e8d5", "0xe169c58d", "0xbc57ac4c", "0x9b00dbd8"]


# -- canonical exponential ------------------------------------------------------

def test_exp_c_accuracy_and_shape():
    # results are flushed to 0 once k = rint(x log2 e) < -125, i.e. x < -86.99
    xs = np.linspace(-86.5, 0.0, 200001).astype(np.float32)
    got = np.array([oracle.exp_c(x) for x in xs], np.float64)
    ref = np.exp(xs.astype(np.float64))
    rel = np.abs(got - ref) / ref
    assert rel.max() < 2.0 ** -21
    assert oracle.exp_c(0.0) == 1.0
    # monotone: non-decreasing in x
    assert np.all(np.diff(got) >= 0)
    for x in np.linspace(-88.0, -86.5, 301).astype(np.float32):
        y = oracle.exp_c(x)
        assert y == 0.0 or (y >= 2.0 ** -126 and abs(y - math.exp(x)) < 2.0 ** -21 * math.exp(x))
    assert oracle.exp_c(-200.0) == 0.0
    assert oracle.exp_c(-1e30) == 0.0


# -- upper bounds of e^x, e^x - 1, tanh(x/2) ------------------------------------

@pytest.mark.parametrize("x", [0.0, 1e-12, 3e-7, 1e-4, 0.01, 0.1234, 0.4999, 0.5, 0.5001,
                               0.9, 1.0, 2.5, 7.0, 20.0, 40.0, 63.9])
def test_bound_functions_dominate_and_are_tight(x):
    L = oracle.lib()
    X = Decimal(x)
    e = X.exp()
    eu = Decimal(L.orc_expu(x))
    assert eu >= e and eu <= e * (1 + Decimal(2) ** -30)
    m = e - 1
    mu = Decimal(L.orc_em1u(x))
    assert mu >= m
    if x > 0:
        assert mu <= m * (1 + Decimal(2) ** -30)
    th = (e - 1) / (e + 1)
    tu = Decimal(L.orc_tanhu(x))
    assert tu >= th
    if x > 0:
        assert tu <= th * (1 + Decimal(2) ** -30) or tu == 1


def test_tv_worst_case_is_tanh():
    """Closed form: for score perturbations confined to [-D, D], the largest
    total variation is reached by the two-level split with mass
    a = 1/(e^D + 1) on the raised side, and equals tanh(D/2)."""
    for D in [1e-3, 0.05, 0.3, 1.0, 3.0]:
        best = 0.0
        for a in np.linspace(1e-4, 1 - 1e-4, 20001):
            w = a * math.exp(D) + (1 - a) * math.exp(-D)
            best = max(best, a * math.exp(D) / w - a)
        a0 = 1 / (math.exp(D) + 1)
        w0 = a0 * math.exp(D) + (1 - a0) * math.exp(-D)
        at = a0 * math.exp(D) / w0 - a0
        assert abs(at - math.tanh(D / 2)) < 1e-12
        assert best <= math.tanh(D / 2) + 1e-12
        assert oracle.lib().orc_tanhu(D) >= math.tanh(D / 2)


def test_fixed_point_rounds_up_and_caps():
    L = oracle.lib()
    assert L.orc_fx(0.0) == 0
    assert L.orc_fx(1.0) == 2 ** 32
    assert L.orc_fx(2.0 ** -33) == 1
    assert L.orc_fx(1.0 + 2.0 ** -40) == 2 ** 32 + 1
    assert L.orc_fx(16383.9) < 2 ** 46
    assert L.orc_fx(16384.0) == 2 ** 46
    assert L.orc_fx(float("inf")) == 2 ** 46


# -- quantization [Meth-1] ------------------------------------------------------

def _k_blocks(rng, d):
    blocks = []
    for kind in range(6):
        k = rng.standard_normal((64, d))
        if kind == 1:
            k[:, : d // 16] *= 10.0
        if kind == 2:
            k[:, 3] = 0.25          # constant channel
            k[:, 5] = 0.0           # zero channel
        if kind == 3:
            k *= 1e-4               # tiny range (subnormal scales)
        if kind == 4:
            k = rng.standard_t(3, (64, d)) * 30.0
        if kind == 5:
            k = np.clip(k * 20000.0, -60000, 60000)
        blocks.append(f16(k))
    return blocks


@pytest.mark.parametrize("d", [64, 128])
def test_int8_key_quantizer_invariants(d):
    rng = np.random.default_rng(3)
    for kb in _k_blocks(rng, d):
        code, s, z = oracle.quant_k_block(kb)
        kf, sf, zf = h2f(kb), h2f(s), h2f(z)
        assert np.array_equal(zf, kf.min(axis=0))                 # offset = exact minimum
        rng_c = kf.max(axis=0) - kf.min(axis=0)
        assert np.all(sf * 255.0 >= rng_c)                        # scale rounded up
        assert np.all((sf == 0) == (rng_c == 0))
        rec = zf[None, :] + sf[None, :] * code.astype(np.float64)
        err = np.abs(kf - rec)
        assert np.all(err <= sf[None, :] * (0.5 + 2.0 ** -14))    # |k - k^| <= kappa s
        # brute force: the code is a nearest level (up to the FP32 rounding slack)
        lv = zf[None, None, :] + sf[None, None, :] * np.arange(256)[:, None, None]
        best = np.abs(kf[None] - lv).min(axis=0)
        assert np.all(err <= best + sf[None, :] * 2.0 ** -14)
        assert np.all(err[:, rng_c == 0] == 0)


@pytest.mark.parametrize("d", [64, 128])
def test_int4_value_quantizer_invariants(d):
    rng = np.random.default_rng(4)
    for vb in _k_blocks(rng, d):
        code, s, z, eta = oracle.quant_v_block(vb)
        vf = h2f(vb)
        lo = code & 15
        hi = code >> 4
        codes = np.empty((64, d), np.int64)
        codes[:, 0::2] = lo
        codes[:, 1::2] = hi
        sf = np.repeat(h2f(s), 32, axis=1)
        zf = np.repeat(h2f(z), 32, axis=1)
        grp = vf.reshape(64, d // 32, 32)
        assert np.array_equal(h2f(z), grp.min(axis=2))
        assert np.all(h2f(s) * 15.0 >= grp.max(axis=2) - grp.min(axis=2))
        rec = zf + sf * codes
        err = np.abs(vf - rec)
        assert np.all(err <= sf * (0.5 + 2.0 ** -14))
        emax = err.max()
        ru = np.float32(emax)
        if float(ru) < emax:
            ru = np.nextafter(ru, np.float32(np.inf))
        assert eta == float(ru)                                   # eta_b = max error, rounded up


@pytest.mark.parametrize("d", [64, 128])
def test_int8_value_quantizer_invariants(d):
    """The symmetric configuration's values: one byte per value, 255 levels
    per (token, 32-channel group); the same invariants as INT4 and a brute
    force nearest-level check; the INT4 codes of the same block are the
    8-bit quantizer's structure at 15 levels (cross-check of the shared
    scale / offset rule)."""
    rng = np.random.default_rng(5)
    for vb in _k_blocks(rng, d):
        code, s, z, eta = oracle.quant_v_block(vb, bits=8)
        assert code.shape == (64, d)
        vf = h2f(vb)
        sf = np.repeat(h2f(s), 32, axis=1)
        zf = np.repeat(h2f(z), 32, axis=1)
        grp = vf.reshape(64, d // 32, 32)
        assert np.array_equal(h2f(z), grp.min(axis=2))
        assert np.all(h2f(s) * 255.0 >= grp.max(axis=2) - grp.min(axis=2))
        rec = zf + sf * code.astype(np.int64)
        err = np.abs(vf - rec)
        assert np.all(err <= sf * (0.5 + 2.0 ** -14))
        lv = zf[None] + sf[None] * np.arange(256)[:, None, None]
        best = np.abs(vf[None] - lv).min(axis=0)
        assert np.all(err <= best + sf * 2.0 ** -14)
        emax = err.max()
        ru = np.float32(emax)
        if float(ru) < emax:
            ru = np.nextafter(ru, np.float32(np.inf))
        assert eta == float(ru)
        # 8-bit steps are (at least) 17x finer than the 4-bit ones
        _, s4, z4, eta4 = oracle.quant_v_block(vb)
        assert np.array_equal(z4, z)
        assert eta <= eta4


# -- scores and the perturbation bound [Meth-2] --------------------------------

def _adversarial_block(rng, d, q):
    """FP16 keys placed 3/8 of a quantization step away from their level, on
    the side of sign(q): the INT8 score error then adds up over channels."""
    s = 2.0 ** -6
    z = -2.0
    k = np.empty((64, d))
    k[0] = z
    k[1] = z + 255 * s
    codes = rng.integers(1, 254, (62, d))
    k[2:] = z + s * (codes + 0.375 * np.sign(h2f(q))[None, :])
    return f16(k)


@pytest.mark.parametrize("d", [64, 128])
def test_delta_dominates_int8_score_error_and_is_tight(d):
    rng = np.random.default_rng(5)
    worst = 0.0
    for trial in range(40):
        q = f16(rng.standard_normal(d) * (1.0 if trial % 2 else 0.1))
        sm = [1.0, 0.125, 0.0883883][trial % 3]
        kb = _adversarial_block(rng, d, q) if trial % 4 == 0 else _k_blocks(rng, d)[trial % 6]
        code, s, z = oracle.quant_k_block(kb)
        sc = oracle.score_q8(q, code, s, z, sm)
        dl, rh = oracle.delta_rho(q, s, z, sm)
        exact = sm * (h2f(kb) @ h2f(q))
        e = np.abs(sc.astype(np.float64) - exact).max()
        assert e <= dl
        worst = max(worst, e / dl)
        s16 = oracle.score_f16(q, kb, sm)
        assert np.abs(s16.astype(np.float64) - exact).max() <= rh
    # the adversarial blocks reach 3/4 of the bound: Delta is not loose by more
    assert worst > 0.7


@pytest.mark.parametrize("d", [64, 128])
def test_int8_score_matches_dequantized_dot_product(d):
    """The INT8 score against the exact dot product with the dequantized keys
    z + s code (FP64): the difference is only the weight and FP rounding,
    E_w + (2^-20 + 2^-23) A + 2^-23 E_w (all of Delta except kappa H)."""
    rng = np.random.default_rng(11)
    for trial in range(30):
        q = f16(rng.standard_normal(d) * 10.0 ** rng.uniform(-3, 1))
        kb = _k_blocks(rng, d)[trial % 6]
        sm = [1.0, 0.125, 0.0883883][trial % 3]
        code, s, z = oracle.quant_k_block(kb)
        sc = oracle.score_q8(q, code, s, z, sm).astype(np.float64)
        qf, sf, zf = h2f(q), h2f(s), h2f(z)
        deq = zf[None, :] + sf[None, :] * code.astype(np.float64)
        exact = sm * (deq @ qf)
        w = (qf * sf).astype(np.float32).astype(np.float64)
        W = np.abs(w).max()
        Ew = 0.0 if W == 0 else 2.0 ** (np.floor(np.log2(W)) - 21) * 255 * d
        A = np.sum(np.abs(qf) * (np.abs(zf) + 255 * sf))
        tol = sm * (Ew + (2.0 ** -20 + 2.0 ** -23) * A + 2.0 ** -23 * Ew) * (1 + 1e-6)
        assert np.abs(sc - exact).max() <= tol, trial
        if W > 0:
            # and the rounding really is small next to the quantization term
            assert tol < 0.05 * sm * 0.5 * np.sum(np.abs(w)) + 1e-30


def test_halving_delta_breaks_dominance():
    """Mutation: with Delta halved in the oracle, the adversarial block's
    INT8 score error exceeds the bound (the dominance check has teeth)."""
    rng = np.random.default_rng(6)
    q = f16(rng.standard_normal(128))
    kb = _adversarial_block(rng, 128, q)
    code, s, z = oracle.quant_k_block(kb)
    sc = oracle.score_q8(q, code, s, z, 1.0)
    exact = h2f(kb) @ h2f(q)
    try:
        oracle.set_mutation(2)
        dl, _ = oracle.delta_rho(q, s, z, 1.0)
    finally:
        oracle.set_mutation(0)
    assert np.abs(sc - exact).max() > dl


def test_block_estimate():
    rng = np.random.default_rng(7)
    for n in [64, 64, 64, 1, 17, 63]:
        sc = (rng.standard_normal(64) * 5).astype(np.float32)
        mx, l = oracle.block_est(sc, n)
        assert mx == sc[:n].max()
        ref = np.exp(sc[:n].astype(np.float64) - mx).sum()
        assert abs(l - ref) / ref < 2.0 ** -19
        assert 1.0 <= l <= n


# -- selection and rank statistic [Meth-3] ---------------------------------------

def test_select_minimal_and_ordered_by_brute_force():
    rng = np.random.default_rng(8)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        m = rng.integers(0, 6, n).astype(np.uint64) * np.uint64(rng.integers(1, 2 ** 30))
        if trial % 3 == 0:
            m = rng.integers(0, 2 ** 38, n).astype(np.uint64)
        total = int(m.sum())
        need = int(rng.integers(0, total + 1)) if total else 0
        k, in_set = oracle.select(m, need)
        if need == 0:
            assert k == 0
            continue
        best = None
        for r in range(1, n + 1):
            if any(sum(int(m[i]) for i in c) >= need for c in itertools.combinations(range(n), r)):
                best = r
                break
        assert k == best
        order = sorted(range(n), key=lambda b: (-int(m[b]), b))
        assert set(np.flatnonzero(in_set)) == set(order[:k])
        assert sum(int(m[b]) for b in order[:k]) >= need


def test_discordant_pairs():
    from scipy.stats import kendalltau
    a = np.arange(10, 0, -1).astype(np.uint64)
    assert oracle.discordant(a, a) == 0
    assert oracle.discordant(a, a[::-1].copy()) == 45
    b = a.copy()
    b[[3, 4]] = b[[4, 3]]
    assert oracle.discordant(a, b) == 1
    rng = np.random.default_rng(9)
    for _ in range(50):
        n = int(rng.integers(2, 60))
        x = rng.permutation(10 * n)[:n].astype(np.uint64)
        y = rng.permutation(10 * n)[:n].astype(np.uint64)
        tau = kendalltau(x.astype(np.int64), y.astype(np.int64)).statistic
        pairs = n * (n - 1) // 2
        assert oracle.discordant(x, y) == round((1 - tau) / 2 * pairs)


def test_dense_head_is_softmax_attention():
    rng = np.random.default_rng(10)
    T, Hkv, d = 300, 2, 64
    k = f16(rng.standard_normal((T, Hkv, d)))
    v = f16(rng.standard_normal((T, Hkv, d)))
    q = f16(rng.standard_normal(d))
    for g in range(Hkv):
        out = oracle.dense_head(k, v, q, g, 0.125)
        s = 0.125 * h2f(k[:, g]) @ h2f(q)
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.abs(out - p @ h2f(v[:, g])).max() < 1e-12

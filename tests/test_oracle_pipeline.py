"""Pins of the oracle's whole decode step on small instances.

The page "Runtime-Certified Bounded-Error Quantized Attention" states the
method's guarantees in words; these tests check them against brute force and
the exact dense result:
  * [Meth-2] the two bounds dominate the measured key and value errors, and
    their sum bounds the distance to exact FP16 attention ([Signif]);
  * [Meth-3] the selected blocks cover tau_cov of the estimated mass with
    the fewest blocks; every rung of the ladder can be reached;
  * [Contrib] a head or layer that falls back returns exactly O_dense.
"""
import numpy as np
import pytest

import datagen
import oracle


def f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def h2f(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def micro(seed, T=512, Hq=4, Hkv=1, d=64, B=1, kind="normal"):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    sm = 1 / np.sqrt(d)
    if kind == "outliers":
        k[..., :4] *= 10
    if kind == "peaked":
        nb = T // 64
        for n in range(B):
            for g in range(Hkv):
                b = int(rng.integers(0, max(nb, 1)))
                u = q[n, g * (Hq // Hkv):(g + 1) * (Hq // Hkv)].mean(0)
                u /= np.linalg.norm(u)
                k[n, b * 64:(b + 1) * 64, g] += 6.0 * u
    if kind == "heavy":
        v = rng.standard_t(3, v.shape)
    if kind == "flat":
        q *= 0.02
    if kind == "big":
        k *= 30
        v *= 50
    return f16(k), f16(v), f16(q), float(sm)


KINDS = ["normal", "outliers", "peaked", "heavy", "flat", "big"]


def certified_heads(res):
    return res.report["rung_max"] < 3


@pytest.mark.parametrize("v_bits", [4, 8])
@pytest.mark.parametrize("seed", range(12))
def test_bounds_dominate_measured_errors(seed, v_bits):
    kind = KINDS[seed % len(KINDS)]
    T = [512, 640, 1000, 200, 64, 130][seed % 6]
    Hq, Hkv = [(4, 1), (8, 2), (2, 2)][seed % 3]
    k, v, q, sm = micro(seed, T=T, Hq=Hq, Hkv=Hkv, kind=kind)
    # tolerances and rank_tol out of reach: every head stays certified
    th = oracle.default_thresholds(sm, k_tol=1e30, v_tol=1e30, rank_tol=1.0)
    r = oracle.certified_decode(k, v, q, th, v_bits=v_bits)
    tr = r.trace
    ok = certified_heads(r)
    assert ok.all()
    ek, ev = tr["bounds"][..., 2], tr["bounds"][..., 3]
    assert np.all(tr["err_key"] <= ek)
    assert np.all(tr["err_val"] <= ev)
    dist = np.abs(r.out - tr["o_dense"]).max(axis=2)
    assert np.all(dist <= ek + ev + 1e-12)
    # reported bounds are the plan's bounds rounded up to FP32
    assert np.all(r.report["e_key"] >= ek) and np.all(r.report["e_val"] >= ev)


@pytest.mark.parametrize("seed", range(6))
def test_symmetric_values_only_change_the_value_term(seed):
    """INT8 values (the symmetric configuration) against INT4 values on the
    same layer: keys, scores, selection, K* and E_key are identical (the
    value width enters nothing on the key side), eta_b and E_val shrink,
    and the output is closer to exact attention in the plain quantized mode."""
    kind = KINDS[seed % len(KINDS)]
    k, v, q, sm = micro(200 + seed, T=[512, 1000, 130][seed % 3], Hq=8, Hkv=2, kind=kind)
    th = oracle.default_thresholds(sm, v_tol=1e30, k_tol=1e30, rank_tol=1.0)
    r4 = oracle.certified_decode(k, v, q, th)
    r8 = oracle.certified_decode(k, v, q, th, v_bits=8)
    for f in ("k_code", "k_s", "k_z", "score", "mfx", "score16"):
        assert np.array_equal(r4.trace[f], r8.trace[f]), f
    assert np.array_equal(r4.trace["sel"] & 1, r8.trace["sel"] & 1)
    assert np.array_equal(r4.report["kstar"], r8.report["kstar"])
    assert np.array_equal(r4.trace["bounds"][..., 2], r8.trace["bounds"][..., 2])
    assert np.all(r8.trace["eta"] <= r4.trace["eta"])
    assert np.all(r8.trace["bounds"][..., 3] <= r4.trace["bounds"][..., 3])
    thn = oracle.default_thresholds(sm, tau_cov=0.0, k_tol=float("inf"), v_tol=float("inf"), rank_tol=1.0)
    n4 = oracle.certified_decode(k, v, q, thn)
    n8 = oracle.certified_decode(k, v, q, thn, v_bits=8)
    d4 = np.abs(n4.out - n4.trace["o_dense"]).max(axis=2)
    d8 = np.abs(n8.out - n8.trace["o_dense"]).max(axis=2)
    assert np.all(d8 <= n8.trace["bounds"][..., 2] + n8.trace["bounds"][..., 3] + 1e-12)
    assert d8.max() <= d4.max()


@pytest.mark.parametrize("seed", range(6))
def test_naive_quantized_mode_is_bounded(seed):
    """tau_cov = 0 with infinite tolerances: no FP16 keys or values (only the
    unfinished block stays exact), the output is plain INT8/INT4 attention,
    and its distance to exact attention is still within E_key + E_val."""
    kind = KINDS[seed % len(KINDS)]
    T = [512, 1000, 130][seed % 3]
    k, v, q, sm = micro(100 + seed, T=T, Hq=8, Hkv=2, kind=kind)
    th = oracle.default_thresholds(sm, tau_cov=0.0, k_tol=float("inf"), v_tol=float("inf"), rank_tol=1.0)
    r = oracle.certified_decode(k, v, q, th)
    assert np.all(r.report["kstar"] == 0) and np.all(r.report["n_v_promoted"] == 0)
    assert np.all(r.report["rung_max"] == 0)
    tr = r.trace
    N = T // 64
    assert not np.any(tr["sel"][..., :N])          # no block of P or VP
    ek, ev = tr["bounds"][..., 2], tr["bounds"][..., 3]
    dist = np.abs(r.out - tr["o_dense"]).max(axis=2)
    assert np.all(dist <= ek + ev + 1e-12)
    # the certified step at the default thresholds is closer to exact
    rc = oracle.certified_decode(k, v, q, oracle.default_thresholds(sm, rank_tol=1.0))
    assert np.abs(rc.out - tr["o_dense"]).max() <= dist.max() + 1e-12


def test_eta_mutation_breaks_value_dominance():
    """Mutation: with eta_b forced to 0 the value bound collapses to 0 while
    the measured INT4 error is not 0: the dominance test has teeth."""
    k, v, q, sm = micro(3, kind="heavy")
    th = oracle.default_thresholds(sm, k_tol=1.0, v_tol=1.0)
    try:
        oracle.set_mutation(1)
        r = oracle.certified_decode(k, v, q, th)
    finally:
        oracle.set_mutation(0)
    assert np.any(r.trace["err_val"] > r.trace["bounds"][..., 3])


def test_coverage_and_minimality():
    """Selected blocks (plus the always-selected partial block) reach
    ceil(tau S) of the fixed-point estimated mass; without widening, dropping
    the smallest selected block falls short (fewest blocks)."""
    tau0 = float(np.float32(0.995))
    for seed, kind in enumerate(KINDS):
        k, v, q, sm = micro(100 + seed, T=1000, Hq=4, Hkv=1, kind=kind)
        th = oracle.default_thresholds(sm, k_tol=1.0, v_tol=1.0)
        r = oracle.certified_decode(k, v, q, th)
        tr = r.trace
        N = 1000 // 64
        for h in range(4):
            M = [int(x) for x in tr["mfx"][0, h]]
            S = sum(M)
            need = int(np.ceil(tau0 * float(S)))
            inP = (tr["sel"][0, h] & 1).astype(bool)
            got = sum(M[b] for b in range(N) if inP[b]) + M[N]
            assert got >= need
            assert r.report["kstar"][0, h] == inP.sum()
            if inP.sum() > 0 and not (r.report["rung_mask"][0, h] & 2):
                smallest = min(M[b] for b in range(N) if inP[b])
                assert got - smallest < need


def test_rung4_reproduces_dense_exactly():
    k, v, q, sm = micro(7, T=640, Hq=8, Hkv=2, kind="outliers")
    th = oracle.default_thresholds(sm, k_tol=-1.0)              # E_key > k_tol always
    r = oracle.certified_decode(k, v, q, th)
    assert np.all(r.report["rung_max"] == 4)
    assert np.all(r.report["rung_mask"] & 2)                    # widened first
    assert np.array_equal(r.out, r.trace["o_dense"])
    assert np.all(r.report["rank_ok"] == -1)
    assert np.all(r.report["e_key"] == 0)


def test_each_rung_can_be_forced():
    k, v, q, sm = micro(8, T=1024, Hq=8, Hkv=2, kind="peaked")
    base = oracle.default_thresholds(sm, k_tol=1.0, v_tol=1.0)
    r = oracle.certified_decode(k, v, q, base)
    assert np.all(r.report["rung_max"] == 0)
    # rung 1: a k_tol that the first plan misses but a wider one meets
    ek = r.trace["bounds"][0, :, 2]
    r1 = oracle.certified_decode(k, v, q, dict(base, k_tol=float(ek.min()) * 0.9))
    assert np.any(r1.report["rung_mask"] & 2)
    # rung 2: v_tol = 0 promotes every value block with a non-zero bound
    r2 = oracle.certified_decode(k, v, q, dict(base, v_tol=0.0))
    assert np.all(r2.report["rung_max"] == 2)
    assert np.all(r2.report["e_val"] == 0)
    assert np.all(r2.trace["err_val"] == 0)
    # rung 2 with too small a cap escalates to rung 4
    r2c = oracle.certified_decode(k, v, q, dict(base, v_tol=0.0, v_cap_blocks=1))
    assert np.all(r2c.report["rung_max"] == 4)
    # rung 3: rank_tol < 0 fails every rank check; f_layer = 1 keeps it per head
    r3 = oracle.certified_decode(k, v, q, dict(base, rank_tol=-1.0, f_layer=1.0))
    assert np.all(r3.report["rung_max"] == 3) and np.all(r3.report["rank_ok"] == 0)
    assert np.array_equal(r3.out, r3.trace["o_dense"])
    # rung 4 after the rank check: more than f_layer of the heads at rung 3
    r4 = oracle.certified_decode(k, v, q, dict(base, rank_tol=-1.0, f_layer=0.5))
    assert np.all(r4.report["rung_max"] == 4) and np.all(r4.report["rung_mask"] & 8)
    assert np.array_equal(r4.out, r4.trace["o_dense"])
    assert np.all(r4.trace["seq_flags"] == 2)


def test_zero_query_selects_first_blocks():
    """q = 0: every score is 0, every block has the same estimated mass, so
    K* = ceil(tau N) and the tie-break picks the first blocks."""
    k, v, q, sm = micro(9, T=1024, Hq=4, Hkv=1)
    q[:] = 0
    r = oracle.certified_decode(k, v, q, oracle.default_thresholds(sm, k_tol=1.0, v_tol=1.0))
    N = 16
    ks = int(np.ceil(np.float64(np.float32(0.995)) * N))
    assert np.all(r.report["kstar"] == ks)
    assert np.all(r.trace["sel"][0, :, :ks] & 1) and not np.any(r.trace["sel"][0, :, ks:] & 1)
    assert np.all(r.trace["score"] == 0)
    assert np.all(r.trace["delta"] == 0)


def test_full_coverage_and_fp16_values_reach_dense():
    """tau = 1 with v_tol = 0: every block with non-zero estimated mass gets
    FP16 keys and FP16 values; the output equals dense attention up to the
    FP32 rounding of the FP16-key scores."""
    k, v, q, sm = micro(10, T=768, Hq=8, Hkv=2, kind="outliers")
    th = oracle.default_thresholds(sm, tau_cov=1.0, k_tol=1.0, v_tol=0.0)
    r = oracle.certified_decode(k, v, q, th)
    assert np.all(r.report["rung_max"] <= 2)
    assert np.abs(r.out - r.trace["o_dense"]).max() < 1e-5


def test_partial_block_is_always_exact_and_in_p():
    k, v, q, sm = micro(11, T=1000, Hq=4, Hkv=1, kind="peaked")
    r = oracle.certified_decode(k, v, q, oracle.default_thresholds(sm, k_tol=1.0, v_tol=1.0))
    tr = r.trace
    assert tr["score"].shape[-1] == 16 * 64
    # the partial block's scores are its FP16-key scores
    sp = oracle.score_f16(q[0, 0], k[0, 960:1000, 0], sm)
    assert np.array_equal(tr["score"][0, 0, 960:1000], sp)
    # its Delta is its rho (no quantization)
    assert np.all(tr["delta"][0, :, 15] == tr["rho"][0, :, 15])


def test_workload_generator_recipe():
    """The plant helper raises the group-mean score by k sigma (analytic)."""
    L = datagen.make_layer("llama_8k", 0, T=4096, Hq=8, Hkv=2)
    info = L.info["plants"]
    G = 4
    for (n, g), pl in info.items():
        qs = h2f(L.q[n, g * G:(g + 1) * G])
        kk = h2f(L.k[n, :, g])
        s = L.sm * kk @ qs.T                     # [T][G]
        blk = s.reshape(-1, 64, G)
        bulk = np.ones(blk.shape[0], bool)
        bulk[pl["random"]] = False
        base = blk[bulk].mean()
        for b in pl["random"]:
            rise = (blk[b].mean() - base) / pl["sigma"]
            assert 3.2 < rise < 4.8
        # sigma estimate matches the bulk score spread
        assert 0.8 < blk[bulk].std() / pl["sigma"] < 1.25

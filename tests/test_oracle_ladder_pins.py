"""Pins of the oracle's ladder pieces that the whole-step tests do not fix.

Each piece is checked against something other than the oracle's own
formula: a layer built so that the answer is known by construction, brute
force over subsets, or the definition written out in numpy.  Each pin also
runs once with a deliberate mistake switched on in the oracle (see
``orc_mutation`` in ckv_oracle.h) and must then fail.

Sources, on the page "Runtime-Certified Bounded-Error Quantized Attention"
(technical summary):
  * rank-consistency check on the promoted blocks: Methodology 3;
  * rung 1 (widen K* to shrink the INT8 tail) and rung 2 (FP16 values for
    the blocks whose estimated value-error contribution is largest):
    Methodology 3, the four-rung fallback ladder;
  * the per-token score perturbation of the unfinished block, which enters
    E_key: Methodology 2.
"""
import itertools

import numpy as np
import pytest
from scipy.stats import kendalltau

import oracle

S6 = 2.0 ** -6    # key quantization step of channel 0 in the rank layers
TOP = 255 * S6    # block maximum of channel 0 (code 255)


@pytest.fixture
def mutation():
    """Switch an oracle mutation on for one block of a test."""
    class M:
        def __init__(self):
            self.flags = 0

        def __call__(self, flags):
            self.flags = flags
            oracle.set_mutation(flags)
            return self

        def __enter__(self):
            return self

        def __exit__(self, *a):
            oracle.set_mutation(0)
    m = M()
    yield m
    oracle.set_mutation(0)


def f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


# ---------------------------------------------------------------------------
# (a) rank-consistency check: a layer whose INT8 and FP16 block orders are
# known by construction
# ---------------------------------------------------------------------------

def rank_layer(peaks, part_peak=None, d=64, seed=0):
    """One kv head, one q head, q = e_0, sm = 1: every score is channel 0
    of the key.  In block b, channel 0 is 0 on every token except token 1
    (TOP = 255/64) and token 2 (the peak (c + e/8)/64, |e| <= 3).  Channel
    0 then quantizes with offset 0 and step 2^-6 exactly, so the INT8 score
    of the peak is c/64 and its FP16 score (c + e/8)/64: the INT8 order of
    the blocks is (c desc, index asc), the FP16 order ((c, e) desc, index
    asc).  The other channels are random (their q is 0).  With part_peak,
    an unfinished block of 10 tokens follows whose token 0 has that score.
    """
    N = len(peaks)
    T = N * 64 + (10 if part_peak is not None else 0)
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((1, T, 1, d))
    v = rng.standard_normal((1, T, 1, d))
    k[0, :, 0, 0] = 0.0
    for b, (c, e) in enumerate(peaks):
        assert 128 <= c <= 254 and abs(e) <= 3
        k[0, b * 64 + 1, 0, 0] = TOP
        k[0, b * 64 + 2, 0, 0] = (c + e / 8) / 64
    if part_peak is not None:
        k[0, N * 64, 0, 0] = part_peak
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    kh, vh, qh = f16(k), f16(v), f16(q)
    # the construction is exact in FP16
    assert np.array_equal(kh.view(np.float16)[0, :, 0, 0].astype(np.float64), k[0, :, 0, 0])
    return kh, vh, qh


def expected_discordant(peaks):
    """Pairs i < j ordered differently: only INT8 ties (equal c) can
    disagree, broken by index in the INT8 order and by e in the FP16 one."""
    D = 0
    for i, j in itertools.combinations(range(len(peaks)), 2):
        (ci, ei), (cj, ej) = peaks[i], peaks[j]
        if ci == cj and ei < ej:
            D += 1
    return D


ALL_IN = dict(tau_cov=1.0, k_tol=float("inf"), v_tol=float("inf"), rank_tol=1.0)


def random_peaks(rng, n, ncodes):
    codes = rng.choice(np.arange(150, 250), size=ncodes, replace=False)
    return [(int(rng.choice(codes)), int(rng.integers(-3, 4))) for _ in range(n)]


RANK_CASES = [
    [(200, 3), (200, -2), (200, 1), (180, 0)],                 # D = 0 + (-2 < 1) = 1
    [(200, -3), (200, -1), (200, 1), (200, 3)],                # ascending e: every pair, D = 6
    [(200, 3), (200, 1), (200, -1), (200, -3)],                # descending e: D = 0
    [(150, 0), (240, 2), (150, 2), (240, -2), (150, -1), (240, 3)],
]


@pytest.mark.parametrize("case", range(len(RANK_CASES) + 6))
def test_rank_check_counts_discordant_pairs_of_a_constructed_layer(case):
    if case < len(RANK_CASES):
        peaks = RANK_CASES[case]
    else:
        rng = np.random.default_rng(100 + case)
        peaks = random_peaks(rng, int(rng.integers(5, 40)), int(rng.integers(1, 5)))
    k, v, q = rank_layer(peaks, part_peak=(None if case % 2 else 7.0), seed=case)
    D = expected_discordant(peaks)
    K = len(peaks)
    if case == 1:
        assert D == 6
    for rank_tol in (1.0, 0.0, 0.2):
        res = oracle.certified_decode(k, v, q, oracle.default_thresholds(1.0, **dict(ALL_IN, rank_tol=rank_tol)))
        r = res.report[0, 0]
        assert r["kstar"] == K
        assert r["n_discordant"] == D, (peaks, r["n_discordant"], D)
        lim = np.floor(np.float32(rank_tol) * (K * (K - 1) / 2))
        assert r["rank_ok"] == int(D <= lim)


def test_rank_check_fp16_masses_closed_form():
    """M16_b = floor(2^32 sum_t exp(s~_t - m)), m the largest FP16-key score
    over P (here TOP), written out in numpy: the unfinished block holds the
    largest INT8-side score (7), which must not enter M16."""
    peaks = [(200, 3), (200, -2), (170, 1), (230, 0), (150, -3)]
    k, v, q = rank_layer(peaks, part_peak=7.0)
    res = oracle.certified_decode(k, v, q, oracle.default_thresholds(1.0, **ALL_IN))
    m16 = res.trace["m16fx"][0, 0].astype(np.float64)
    for b, (c, e) in enumerate(peaks):
        s = np.zeros(64)
        s[1] = TOP
        s[2] = (c + e / 8) / 64
        want = np.exp(s - TOP).sum() * 2.0 ** 32
        assert abs(m16[b] - want) <= 1e-6 * want, (b, m16[b], want)


def test_rank_check_matches_kendall_tau_on_random_layers():
    """On random layers with large promoted sets, the reported discordant
    count equals the one scipy's Kendall tau gives for the exported INT8
    and FP16 masses over P with the (mass desc, index asc) keys."""
    rng = np.random.default_rng(5)
    for it in range(4):
        T, d, Hq = [640, 1280, 960, 2048][it], [64, 128][it % 2], 4
        k = rng.standard_normal((1, T, 1, d))
        v = rng.standard_normal((1, T, 1, d))
        q = rng.standard_normal((1, Hq, d)) * 0.05
        res = oracle.certified_decode(f16(k), f16(v), f16(q),
                                      oracle.default_thresholds(1 / np.sqrt(d), tau_cov=1.0, rank_tol=1.0))
        tr = res.trace
        for h in range(Hq):
            P = np.nonzero(tr["sel"][0, h] & 1)[0]
            K = len(P)
            assert K == res.report[0, h]["kstar"] and K >= 8
            ki = [(int(tr["mfx"][0, h, b]) << 16) | (0xFFFF - int(b)) for b in P]
            k16 = [(int(tr["m16fx"][0, h, b]) << 16) | (0xFFFF - int(b)) for b in P]
            # unique keys: tau = (C - D) / (C + D), C + D = K (K - 1) / 2;
            # the 54-bit keys go to scipy as exact ranks (Python int sort)
            def ranks(keys):
                r = np.empty(len(keys), np.int64)
                r[sorted(range(len(keys)), key=lambda i: keys[i])] = np.arange(len(keys))
                return r
            tau = kendalltau(ranks(ki), ranks(k16)).statistic
            pairs = K * (K - 1) // 2
            D = int(round((1 - tau) * pairs / 2))
            assert res.report[0, h]["n_discordant"] == D, (it, h)


@pytest.mark.parametrize("flags", [4, 16])
def test_rank_check_pin_fails_under_mutation(flags, mutation):
    peaks = RANK_CASES[0] + RANK_CASES[3]
    k, v, q = rank_layer(peaks, part_peak=7.0)
    D = expected_discordant(peaks)
    with mutation(flags):
        res = oracle.certified_decode(k, v, q, oracle.default_thresholds(1.0, **ALL_IN))
    assert res.report[0, 0]["n_discordant"] != D


def test_rank_fp16_mass_pin_fails_under_mutation(mutation):
    with mutation(8):
        with pytest.raises(AssertionError):
            test_rank_check_fp16_masses_closed_form()


# ---------------------------------------------------------------------------
# (b) rung 2: VP is the fewest blocks by (contribution desc, index asc)
# ---------------------------------------------------------------------------

def fx_bound(u):
    """A fixed-point sum (2^-32 units) as the bound it stands for, rounded up."""
    return float(u) * 2.0 ** -32 * (1.0 + 2.0 ** -50)


def rung2_instance(seed, n_vp):
    """12 blocks, peaked attention; v_tol set between the rest sums after
    promoting n_vp - 1 and n_vp blocks by descending contribution."""
    rng = np.random.default_rng(seed)
    T, d, Hq = 12 * 64, 64, 2
    k = rng.standard_normal((1, T, 1, d))
    v = rng.standard_normal((1, T, 1, d)) * (1 + 3 * rng.random((1, T, 1, 1)))
    q = rng.standard_normal((1, Hq, d))
    for j in range(3):
        b = int(rng.integers(0, 12))
        k[0, b * 64:(b + 1) * 64, 0] += (1.5 + j) * q[0, j % Hq] / np.linalg.norm(q[0, j % Hq])
    k, v, q = f16(k), f16(v), f16(q)
    sm = 1 / np.sqrt(d)
    base = oracle.certified_decode(k, v, q, oracle.default_thresholds(sm, v_tol=float("inf")))
    tols = []
    for h in range(Hq):
        cv = sorted((int(x) for x in base.trace["cval"][0, h]), reverse=True)
        lo, hi = fx_bound(sum(cv[n_vp:])), fx_bound(sum(cv[n_vp - 1:]))
        tols.append((lo, hi))
    # one v_tol for both heads inside both windows when they overlap, else
    # the first head's window (the second head is then checked as it comes)
    lo = max(t[0] for t in tols)
    hi = min(t[1] for t in tols)
    vt = np.float32((lo + hi) / 2) if lo < hi else np.float32((tols[0][0] + tols[0][1]) / 2)
    return k, v, q, sm, float(vt)


def check_rung2(res, v_tol):
    tr = res.trace
    for h in range(res.report.shape[1]):
        cv = [int(x) for x in tr["cval"][0, h]]
        N = len(cv)
        vp = set(np.nonzero(tr["sel"][0, h] & 2)[0].tolist())
        nvp = res.report[0, h]["n_v_promoted"]
        assert len(vp) == nvp
        order = sorted(range(N), key=lambda b: (-cv[b], b))
        # VP is a prefix of (contribution desc, index asc)
        assert vp == set(order[:nvp]), (h, sorted(vp), order[:nvp])
        rest = sum(cv[b] for b in range(N) if b not in vp)
        assert tr["bounds"][0, h, 3] == fx_bound(rest)
        assert fx_bound(rest) <= v_tol
        # and no smaller set of blocks reaches v_tol (brute force)
        for m in range(nvp):
            for W in itertools.combinations(range(N), m):
                assert fx_bound(sum(cv) - sum(cv[b] for b in W)) > v_tol, (h, W)


@pytest.mark.parametrize("seed,n_vp", [(1, 2), (2, 3), (3, 4), (4, 1), (5, 6)])
def test_rung2_promotes_fewest_blocks_by_contribution(seed, n_vp):
    k, v, q, sm, vt = rung2_instance(seed, n_vp)
    res = oracle.certified_decode(k, v, q, oracle.default_thresholds(sm, v_tol=vt))
    assert res.report[0]["n_v_promoted"].max() >= 1
    check_rung2(res, vt)


def test_rung2_pin_fails_under_mutation(mutation):
    k, v, q, sm, vt = rung2_instance(2, 3)
    with mutation(32):
        res = oracle.certified_decode(k, v, q, oracle.default_thresholds(sm, v_tol=vt))
    with pytest.raises(AssertionError):
        check_rung2(res, vt)


# ---------------------------------------------------------------------------
# (c) rung 1: each widening halves the uncovered target 1 - tau, and the
# widening stops at the first tau whose E_key meets k_tol
# ---------------------------------------------------------------------------

def tau_after(tau0, w):
    t = float(np.float32(tau0))
    for _ in range(w):
        t = 1.0 - (1.0 - t) * 0.5
    return t


def rung1_layer(seed):
    rng = np.random.default_rng(seed)
    T, d, Hq = 2048 + 37, 64, 4
    k = rng.standard_normal((1, T, 1, d))
    v = rng.standard_normal((1, T, 1, d))
    q = rng.standard_normal((1, Hq, d)) * 0.6
    return f16(k), f16(v), f16(q), 1 / np.sqrt(d)


def check_rung1(k, v, q, sm, k_tol, n_widen=3):
    th = oracle.default_thresholds(sm, k_tol=k_tol, n_widen=n_widen, v_tol=float("inf"))
    res = oracle.certified_decode(k, v, q, th)
    tr = res.trace
    N = k.shape[1] // 64
    widened = 0
    for h in range(q.shape[1]):
        r = res.report[0, h]
        ws = [w for w in range(n_widen + 1) if np.float32(tau_after(th["tau_cov"], w)) == r["tau_final"]]
        assert len(ws) == 1, (h, r["tau_final"])
        w = ws[0]
        assert bool(r["rung_mask"] & 2) == (w > 0)
        widened += w > 0
        # P is the selection at the final tau (orc_select on the exported masses)
        M = tr["mfx"][0, h]
        S = int(M.sum(dtype=np.uint64))
        need = int(np.ceil(tau_after(th["tau_cov"], w) * float(S))) - int(M[N])
        kst, in_set = oracle.select(M[:N], max(need, 0))
        assert kst == r["kstar"] and np.array_equal(in_set, tr["sel"][0, h] & 1)
        # E_key meets k_tol at w unless the cap was reached; with one
        # widening fewer allowed, the cap is reached (escalation to rung 4)
        if w < n_widen:
            assert tr["bounds"][0, h, 2] <= k_tol
        if w > 0:
            r2 = oracle.certified_decode(k, v, q, dict(th, n_widen=w - 1), trace=False).report[0, h]
            assert r2["rung_mask"] & 16 and r2["tau_final"] == np.float32(tau_after(th["tau_cov"], w - 1))
    return widened


@pytest.mark.parametrize("seed", [0, 1])
def test_rung1_halves_the_uncovered_target(seed):
    k, v, q, sm = rung1_layer(seed)
    base = oracle.certified_decode(k, v, q, oracle.default_thresholds(sm, k_tol=float("inf"), v_tol=float("inf")))
    ek = np.sort(base.trace["bounds"][0, :, 2])
    # k_tol just below the second-largest E_key at tau0: at least two heads widen
    widened = check_rung1(k, v, q, sm, float(np.float32(ek[-2] * 0.6)))
    assert widened >= 2


def test_rung1_pin_fails_under_mutation(mutation):
    k, v, q, sm = rung1_layer(0)
    base = oracle.certified_decode(k, v, q, oracle.default_thresholds(sm, k_tol=float("inf"), v_tol=float("inf")))
    ek = np.sort(base.trace["bounds"][0, :, 2])
    with mutation(64):
        with pytest.raises(AssertionError):
            check_rung1(k, v, q, sm, float(np.float32(ek[-2] * 0.6)))


# ---------------------------------------------------------------------------
# (d) rho of the unfinished block: sm 2^-23 A (1 + 2^-20), A = sum_c |q_c|
# max_t |k_tc|, rounded up to FP32; and it bounds the FP16-key score error
# ---------------------------------------------------------------------------

def rho_partial_expected(kp, qh, sm):
    A = float(np.sum(np.abs(qh) * np.abs(kp).max(axis=0)))
    return float(sm) * 2.0 ** -23 * A * (1 + 2.0 ** -20)


def check_rho_partial(seeds=range(6)):
    for seed in seeds:
        rng = np.random.default_rng(seed)
        d = [64, 128][seed % 2]
        np_ = int(rng.integers(1, 64))
        T = 64 * int(rng.integers(0, 4)) + np_
        k = rng.standard_normal((1, T, 1, d)) * rng.choice([1.0, 30.0])
        k[..., :3] -= 4.0          # channels whose largest |k| is a negative key
        v = rng.standard_normal((1, T, 1, d))
        q = rng.standard_normal((1, 2, d))
        kh, vh, qh = f16(k), f16(v), f16(q)
        sm = float(np.float32(1 / np.sqrt(d)))   # the thresholds hold sm in FP32
        res = oracle.certified_decode(kh, vh, qh, oracle.default_thresholds(sm))
        N = T // 64
        kp = kh.view(np.float16)[0, N * 64:, 0].astype(np.float64)
        for h in range(2):
            qv = qh.view(np.float16)[0, h].astype(np.float64)
            rho = res.trace["rho"][0, h, N]
            want = rho_partial_expected(kp, qv, sm)
            # rounded up to FP32: the smallest float >= want, up to the
            # rounding of numpy's sum order (one float step)
            assert want <= float(rho) * (1 + 1e-12)
            assert float(np.nextafter(rho, np.float32(0))) < want * (1 + 1e-12)
            assert res.trace["delta"][0, h, N] == rho
            # the FP16-key scores of the unfinished block are within rho of
            # the exact scores
            ex = (kp @ qv) * sm
            sc = res.trace["score"][0, h, N * 64:N * 64 + np_].astype(np.float64)
            assert np.all(np.abs(sc - ex) <= rho)


def test_rho_of_unfinished_block_matches_definition():
    check_rho_partial()


def test_rho_pin_fails_under_mutation(mutation):
    with mutation(128):
        with pytest.raises(AssertionError):
            check_rho_partial()

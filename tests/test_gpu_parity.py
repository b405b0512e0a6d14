"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bit-exact: quantized codes, scales, offsets and eta_b; INT8 scores, block
estimates, Delta, rho; fixed-point masses; selected sets P and VP; the FP64
bounds; rank verdicts and discordant counts; rungs.  Outputs: within
2e-3 absolute + 1e-2 relative of the oracle (FP32 accumulation on the GPU,
FP64 in the oracle).
"""
import zlib

import numpy as np
import pytest

import datagen
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import certified_quantized_kv_amd as ckv  # noqa: F401  (raises if the library is missing)


def f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def make_cache(B, Hq, Hkv, d, T, v_bits=4):
    import certified_quantized_kv_amd as ckv
    return ckv.Cache(1, B, Hq, Hkv, d, T, v_bits=v_bits)


def gpu_run(k, v, q, th, chunks=None, cache=None, v_bits=4):
    """Append k, v ([B][T][Hkv][d] uint16) and run one decode step."""
    B, T, Hkv, d = k.shape
    Hq = q.shape[1]
    c = cache or make_cache(B, Hq, Hkv, d, T, v_bits=v_bits)
    for n in range(B):
        if chunks is None:
            c.append_kv(0, n, k[n], v[n])
        else:
            t0 = 0
            for i, ln in enumerate(chunks):
                kk = k[n, t0:t0 + ln]
                vv = v[n, t0:t0 + ln]
                if i % 2:   # every other chunk from device memory
                    c.append_kv(0, n, torch.from_numpy(kk.view(np.float16)).cuda(),
                                torch.from_numpy(vv.view(np.float16)).cuda())
                else:
                    c.append_kv(0, n, kk, vv)
                t0 += ln
            assert t0 == T
    qd = torch.from_numpy(q.view(np.float16)).cuda()
    out, rep = c.certified_decode_attention(0, qd, th)
    torch.cuda.synchronize()
    step = c.export_step(B)
    return c, out.cpu().numpy().astype(np.float64), rep, step


def check_parity(k, v, q, th, res, c, out, rep, step):
    """Compare the GPU step with the oracle result `res` on every sequence
    and head of the batch."""
    B, T, Hkv, d = k.shape
    Hq = q.shape[1]
    G = Hq // Hkv
    N = T // 64
    tr = res.trace
    for n in range(B):
        oi = n
        # tier 1, bit-exact
        for og, g in enumerate(range(Hkv)):
            for b in sorted({0, N // 2, N - 1} if N else set()):
                e = c.export_block(0, n, g, b)
                assert np.array_equal(e["k_code"], tr["k_code"][oi, og, b]), (n, g, b)
                assert np.array_equal(e["k_s"], tr["k_s"][oi, og, b])
                assert np.array_equal(e["k_z"], tr["k_z"][oi, og, b])
                assert np.array_equal(e["v_code"], tr["v_code"][oi, og, b])
                assert np.array_equal(e["v_s"], tr["v_s"][oi, og, b])
                assert np.array_equal(e["v_z"], tr["v_z"][oi, og, b])
                assert e["eta"][0] == tr["eta"][oi, og, b]
        Np = tr["score"].shape[-1] // 64
        for oh, h in enumerate(range(Hq)):
            g, j = h // G, h % G
            ctx = (n, h)
            assert np.array_equal(step["score"][n, h, :Np * 64], tr["score"][oi, oh]), ctx
            bs = step["bstat"][n, h, :Np]
            assert np.array_equal(bs[:, 0], tr["bmax"][oi, oh]), ctx
            assert np.array_equal(bs[:, 1], tr["bl"][oi, oh]), ctx
            assert np.array_equal(bs[:, 2], tr["delta"][oi, oh]), ctx
            assert np.array_equal(bs[:, 3], tr["rho"][oi, oh]), ctx
            assert step["mref"][n, h] == tr["mref"][oi, oh], ctx
            assert np.array_equal(step["mfx"][n, h, :Np], tr["mfx"][oi, oh]), ctx
            sel = step["sel"][n, g, :N]
            assert np.array_equal((sel >> j) & 1, tr["sel"][oi, oh] & 1), ctx
            assert np.array_equal((sel >> (8 + j)) & 1, (tr["sel"][oi, oh] >> 1) & 1), ctx
            assert np.array_equal(step["bounds"][n, h], tr["bounds"][oi, oh]), ctx
            ro, rg = res.report[oi, oh], rep[n, h]
            for f in ("kstar", "n_v_promoted", "tau_final"):
                assert ro[f] == rg[f], (ctx, f, ro[f], rg[f])
        # the ladder outcome (per sequence and layer)
        assert step["seq_flags"][n] == tr["seq_flags"][oi], n
        for h in range(Hq):
            ro, rg = res.report[oi, h], rep[n, h]
            for f in ("rank_ok", "n_discordant", "rung_max", "rung_mask", "e_key", "e_val",
                      "tv_bound"):
                assert ro[f] == rg[f], ((n, h), f, ro[f], rg[f])
            if not (tr["seq_flags"][oi] & 1):
                inP = (tr["sel"][oi, h] & 1).astype(bool)
                assert np.array_equal(step["m16fx"][n, h, :N][inP], tr["m16fx"][oi, h][inP]), (n, h)
        ref = res.out[oi]
        assert np.all(np.abs(out[n] - ref) <= ATOL + RTOL * np.abs(ref)), \
            (n, np.abs(out[n] - ref).max())


def both(k, v, q, th, chunks=None, v_bits=4):
    print(f"case B={k.shape[0]} T={k.shape[1]} Hkv={k.shape[2]} d={k.shape[3]} Hq={q.shape[1]} "
          f"v_bits={v_bits} th={th}", flush=True)
    res = oracle.certified_decode(k, v, q, th, v_bits=v_bits)
    c, out, rep, step = gpu_run(k, v, q, th, chunks=chunks, v_bits=v_bits)
    check_parity(k, v, q, th, res, c, out, rep, step)
    c.close()
    return res, rep


def micro(seed, T=512, Hq=4, Hkv=1, d=64, B=1, kind="normal"):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    if kind == "outliers":
        k[..., :4] *= 10
    if kind == "peaked":
        for n in range(B):
            for g in range(Hkv):
                b = int(rng.integers(0, max(T // 64, 1)))
                u = q[n, g * (Hq // Hkv):(g + 1) * (Hq // Hkv)].mean(0)
                k[n, b * 64:(b + 1) * 64, g] += 6.0 * u / np.linalg.norm(u)
    if kind == "heavy":
        v = rng.standard_t(3, v.shape)
    if kind == "flat":
        q *= 0.02
    return f16(k), f16(v), f16(q), float(1 / np.sqrt(d))


# -- small cases: every intermediate ------------------------------------------

THRESHOLD_CASES = [
    dict(),                                       # defaults
    dict(v_cap_blocks=1),                         # rung 2 cap -> rung 4 before paging
    dict(rank_tol=-1.0, f_layer=1.0),             # rung 3 on every head
    dict(rank_tol=-1.0, f_layer=0.5),             # rung 4 after the rank check
    dict(k_tol=2e-4),                             # rung 1 widening
    dict(tau_cov=1.0, v_tol=0.0, k_tol=1.0),      # everything promoted
    dict(tau_cov=0.0, k_tol=float("inf"), v_tol=float("inf")),   # plain INT8/INT4 attention
]


@pytest.mark.parametrize("case", range(len(THRESHOLD_CASES)))
def test_tiny_config_all_rungs(case):
    L = datagen.make_layer("tiny_1k", 0)
    th = oracle.default_thresholds(L.sm, **THRESHOLD_CASES[case])
    both(L.k, L.v, L.q, th)


@pytest.mark.parametrize("chunks", [None, [1, 63, 100, 500, 336], [1000], [64, 64, 872]])
def test_ragged_context_and_chunked_appends(chunks):
    L = datagen.make_layer("tiny_1k", 0, T=1000)
    th = oracle.default_thresholds(L.sm)
    both(L.k, L.v, L.q, th, chunks=chunks)


@pytest.mark.parametrize("shape", [(4, 1, 64), (8, 2, 64), (2, 2, 64), (16, 2, 128), (8, 1, 128),
                                   (4, 4, 128)])
@pytest.mark.parametrize("kind", ["normal", "peaked", "heavy", "flat", "outliers"])
def test_head_shapes_and_distributions(shape, kind):
    Hq, Hkv, d = shape
    seed = zlib.crc32(repr((shape, kind)).encode()) % 1000
    k, v, q, sm = micro(seed, T=[640, 1000, 130][seed % 3], Hq=Hq, Hkv=Hkv, d=d, B=2, kind=kind)
    both(k, v, q, oracle.default_thresholds(sm))


@pytest.mark.parametrize("case", range(len(THRESHOLD_CASES)))
def test_symmetric_cache_tiny_config_all_rungs(case):
    """INT8 values (the symmetric cache configuration): codes, eta_b and every
    intermediate and output against the oracle run at 8-bit values."""
    L = datagen.make_layer("tiny_1k", 0)
    th = oracle.default_thresholds(L.sm, **THRESHOLD_CASES[case])
    both(L.k, L.v, L.q, th, v_bits=8)


@pytest.mark.parametrize("shape", [(4, 1, 64), (8, 2, 64), (16, 2, 128), (8, 1, 128)])
@pytest.mark.parametrize("kind", ["normal", "heavy", "flat"])
def test_symmetric_cache_head_shapes(shape, kind):
    Hq, Hkv, d = shape
    seed = zlib.crc32(repr((shape, kind, 8)).encode()) % 1000
    k, v, q, sm = micro(seed, T=[640, 1000, 130][seed % 3], Hq=Hq, Hkv=Hkv, d=d, B=2, kind=kind)
    both(k, v, q, oracle.default_thresholds(sm, tau_cov=0.0, k_tol=float("inf"), v_tol=float("inf")),
         v_bits=8)
    both(k, v, q, oracle.default_thresholds(sm), v_bits=8)


def planted_excess(seed, A=96.0, T=512 + 17, d=64, Hq=2):
    """A layer where a P block's FP16-key scores exceed the largest INT8
    block estimate M^ by more than ln 4: one token of block 3 has every
    channel 0.4 of a quantization step past a rounding point, against the
    sign of q_c, so its INT8 score is low by about 0.8 Delta (Delta ~ 2
    with keys spanning [-A, A] in every channel of the block) while it is
    the largest exact score.  Both q heads are equal."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, Hq, d))
    q[0, 1:] = q[0, 0]
    k = rng.uniform(-0.5, 0.5, (1, T, 1, d)) * A
    v = rng.standard_normal((1, T, 1, d))
    blk = k[0, 3 * 64:4 * 64, 0]
    blk[0], blk[1] = -A, A
    s = 2 * A / 255
    sg = np.sign(q[0, 0])
    blk[21] = -A + (np.where(sg > 0, 230, 25) + np.where(sg > 0, 0.4, -0.4)) * s
    return f16(k), f16(v), f16(q), float(1 / np.sqrt(d))


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("v_tol", [float("inf"), 0.0])
def test_promoted_weights_when_fp16_key_scores_exceed_the_estimate(seed, v_tol):
    """The promoted value passes weigh FP16-key scores, which may exceed
    M^ by up to Delta + rho; their softmax reference must cover that
    (weights above 4 would overflow the FP16 operands of the value
    contraction).  INT4 values (v_tol = inf) and FP16 values (v_tol = 0);
    the rank check never fails (rank_tol = 1), so the promoted passes give
    the output."""
    k, v, q, sm = planted_excess(seed)
    th = oracle.default_thresholds(sm, k_tol=float("inf"), v_tol=v_tol, rank_tol=1.0)
    res, rep = both(k, v, q, th)
    tr = res.trace
    N = k.shape[1] // 64
    for h in range(q.shape[1]):
        inP = (tr["sel"][0, h] & 1).astype(bool)
        s16 = tr["score16"][0, h, :N * 64].reshape(N, 64)[inP]
        assert s16.max() - tr["mref"][0, h] > np.log(4.0) + 0.05
        assert rep[0, h]["rung_max"] == (2 if v_tol == 0.0 else 0)


def test_single_token_and_single_block():
    for T in [1, 63, 64, 65]:
        k, v, q, sm = micro(T, T=T, Hq=8, Hkv=2, d=128)
        both(k, v, q, oracle.default_thresholds(sm))


@pytest.mark.parametrize("nblk", [513, 700, 1024, 1500, 2048])
def test_rank_check_large_promoted_sets(nblk):
    """K* above the direct-pairs limit: the sorted rank check (bitonic sort of
    the INT8 order, merge count of the FP16 order) against the oracle."""
    k, v, q, sm = micro(900 + nblk, T=64 * nblk, Hq=4, Hkv=1, d=64, kind="flat")
    th = oracle.default_thresholds(sm, tau_cov=1.0, rank_tol=1.0)
    res, rep = both(k, v, q, th)
    assert np.all(rep["kstar"] == nblk)
    assert np.all(rep["n_discordant"] > 0)


def test_batch_with_some_sequences_at_rung4_before_paging():
    """A batch whose sequences differ in how many FP16 value blocks they ask
    for: with a small cap, sequences 1 and 3 (values of unit range, flat
    attention) go to rung 4 before paging, so their lists count as empty in
    the passes that split the whole step's lists, while sequences 0 and 2
    (values of small range) are certified; every intermediate against the
    oracle."""
    rng = np.random.default_rng(77)
    B, T, Hq, Hkv, d = 4, 1280, 8, 4, 64
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    v[0] *= 0.01
    v[2] *= 0.01
    q[1] *= 0.02
    q[3] *= 0.02
    th = oracle.default_thresholds(1 / np.sqrt(d), v_cap_blocks=2)
    res, rep = both(f16(k), f16(v), f16(q), th)
    assert list(res.trace["seq_flags"] & 1) == [0, 1, 0, 1]


@pytest.mark.parametrize("staged", [True, False])
def test_batch_with_skipped_sequences_and_rung3_heads(staged):
    """Rung 4 before paging on sequences 1 and 3 (a small cap) and rung 3 on
    every head of sequences 0 and 2 (rank_tol < 0, f_layer = 1) in one step:
    the dense pass then reads the skipped sequences' blocks (all listed at
    the end of the packed staging areas) and the rung-3 pairs' blocks (those
    of the first listing and the ones the fallback adds), through the slot
    maps with staged paging, by (pair, block) with run copies; every
    intermediate and output against the oracle, two layers in a row."""
    import certified_quantized_kv_amd as ckv
    rng = np.random.default_rng(78)
    B, T, Hq, Hkv, d = 4, 1280 + 37, 8, 4, 64
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    v[0] *= 0.01
    v[2] *= 0.01
    q[1] *= 0.02
    q[3] *= 0.02
    k, v, q = f16(k), f16(v), f16(q)
    th = oracle.default_thresholds(1 / np.sqrt(d), v_cap_blocks=2, rank_tol=-1.0, f_layer=1.0)
    res = oracle.certified_decode(k, v, q, th)
    assert list(res.trace["seq_flags"] & 1) == [0, 1, 0, 1]
    assert np.all(res.report["rung_max"][[0, 2]] == 3) and np.all(res.report["rung_max"][[1, 3]] == 4)
    c = ckv.Cache(2, B, Hq, Hkv, d, T)
    if not staged:
        c.set_staged_paging(0)
    for l in range(2):
        for n in range(B):
            c.append_kv(l, n, k[n], v[n])
    qd = torch.from_numpy(q.view(np.float16)).cuda()
    for l in range(2):
        out, rep = c.certified_decode_attention(l, qd, th)
        torch.cuda.synchronize()
        for f in ("kstar", "n_v_promoted", "rank_ok", "n_discordant", "rung_max", "rung_mask", "e_key",
                  "e_val", "tv_bound", "tau_final"):
            assert np.array_equal(res.report[f], rep[f]), (l, f)
        o = out.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(o - res.out) <= ATOL + RTOL * np.abs(res.out)), (l, np.abs(o - res.out).max())
    c.close()


def test_mixed_lengths_in_a_batch():
    """Sequences of different lengths in one step (each compared alone)."""
    import certified_quantized_kv_amd as ckv
    Hq, Hkv, d = 8, 2, 128
    lens = [1000, 256, 70]
    c = ckv.Cache(1, 3, Hq, Hkv, d, 1024)
    ks, vs = [], []
    for n, T in enumerate(lens):
        k, v, q, sm = micro(50 + n, T=T, Hq=Hq, Hkv=Hkv, d=d)
        c.append_kv(0, n, k[0], v[0])
        ks.append(k)
        vs.append(v)
    rng = np.random.default_rng(3)
    q = f16(rng.standard_normal((3, Hq, d)))
    th = oracle.default_thresholds(sm)
    out, rep = c.certified_decode_attention(0, torch.from_numpy(q.view(np.float16)).cuda(), th)
    out = out.cpu().numpy()
    for n, T in enumerate(lens):
        res = oracle.certified_decode(ks[n], vs[n], q[n:n + 1], th)
        for f in ("kstar", "n_v_promoted", "rung_mask", "e_key", "e_val", "n_discordant"):
            assert np.array_equal(rep[n][f], res.report[0][f]), (n, f)
        ref = res.out[0]
        assert np.all(np.abs(out[n] - ref) <= ATOL + RTOL * np.abs(ref))
    c.close()


def test_steps_with_fewer_sequences_than_the_cache_holds():
    """Steps over the first 2, then all 4, then the first 1 of a cache made
    for 4 sequences: the selection and the plans reach the host for the
    step's own batch only, and what a larger earlier step left there is
    never read (every step compared with the oracle on each sequence)."""
    import certified_quantized_kv_amd as ckv
    Hq, Hkv, d, T = 8, 2, 128, 1000
    k, v, q, sm = micro(61, T=T, Hq=Hq, Hkv=Hkv, d=d, B=4, kind="peaked")
    th = oracle.default_thresholds(sm)
    c = ckv.Cache(1, 4, Hq, Hkv, d, T)
    for n in range(4):
        c.append_kv(0, n, k[n], v[n])
    for batch in (2, 4, 1):
        print(f"case batch {batch} of 4", flush=True)
        out, rep = c.certified_decode_attention(0, torch.from_numpy(q[:batch].view(np.float16)).cuda(), th)
        out = out.cpu().numpy()
        res = oracle.certified_decode(k[:batch], v[:batch], q[:batch], th)
        for f in ("kstar", "n_v_promoted", "rank_ok", "n_discordant", "rung_max", "rung_mask", "e_key",
                  "e_val", "tv_bound", "tau_final"):
            assert np.array_equal(rep[f], res.report[f]), (batch, f)
        assert np.all(np.abs(out - res.out) <= ATOL + RTOL * np.abs(res.out)), batch
    c.close()


def test_deterministic_across_runs():
    L = datagen.make_layer("tiny_1k", 0, T=1000)
    th = oracle.default_thresholds(L.sm)
    c, out1, rep1, s1 = gpu_run(L.k, L.v, L.q, th)
    qd = torch.from_numpy(L.q.view(np.float16)).cuda()
    out2, rep2 = c.certified_decode_attention(0, qd, th)
    s2 = c.export_step(1)
    assert np.array_equal(out1, out2.cpu().numpy().astype(np.float64))
    assert np.array_equal(rep1, rep2)
    for key in s1:
        assert np.array_equal(s1[key], s2[key]), key
    c.close()


# -- full-size workloads ---------------------------------------------------------

def test_llama_8k_layer():
    L = datagen.make_layer("llama_8k", 0)
    both(L.k, L.v, L.q, oracle.default_thresholds(L.sm))


def test_llama_8k_layer_symmetric_cache():
    """The full 8K layer with 8-bit values (the symmetric configuration)."""
    L = datagen.make_layer("llama_8k", 1)
    both(L.k, L.v, L.q, oracle.default_thresholds(L.sm), v_bits=8)


# The rungs each stress layer is built to reach (the workload's layer
# variants): the oracle and the GPU must both reach them, so a drift of the
# generator cannot silently drop rung-3/4 coverage at full size.
STRESS_RUNGS = {
    0: dict(mask_all=0b1110, seq_flags=0, min_rung3=1),    # rungs 1, 2 and 3 on flipped pairs
    1: dict(mask_all=0b11110, seq_flags=2, min_rung3=17),  # > half the heads at rung 3 -> rung 4
    2: dict(mask_all=0b1110, seq_flags=0, min_rung3=1),    # rung 3 on the flat-copy group
    3: dict(mask_all=0b0100, seq_flags=0, min_rung3=0),    # certifies with rung 2
}


@pytest.mark.parametrize("layer", [0, 1, 2, 3])
def test_stress_32k_layers(layer):
    L = datagen.make_layer("stress_32k", layer)
    res, rep = both(L.k, L.v, L.q, oracle.default_thresholds(L.sm))
    want = STRESS_RUNGS[layer]
    for r in (res.report[0], rep[0]):
        assert np.bitwise_or.reduce(r["rung_mask"]) == want["mask_all"], layer
        assert int(np.sum(r["rank_ok"] == 0)) >= want["min_rung3"], layer
    assert res.trace["seq_flags"][0] == want["seq_flags"]
    if want["seq_flags"] & 2:
        assert np.all(rep[0]["rung_max"] == 4)


def full_layer(name, layer):
    """A full layer of a workload on the GPU against the oracle on every
    sequence and head: tier 1, every intermediate, the ladder outcome
    (rank verdicts, discordant counts, rungs, reported bounds, FP16-side
    masses) and the outputs."""
    L = datagen.make_layer(name, layer)
    th = oracle.default_thresholds(L.sm)
    print(f"case {name} layer {layer}", flush=True)
    res = oracle.certified_decode(L.k, L.v, L.q, th)
    c, out, rep, step = gpu_run(L.k, L.v, L.q, th)
    check_parity(L.k, L.v, L.q, th, res, c, out, rep, step)
    c.close()
    return res, rep


def test_llama_32k_batch4_layer0():
    """Full 4 x 32K layer, all four sequences."""
    full_layer("llama_32k", 0)


def test_needle_64k_layer0():
    full_layer("needle_64k", 0)


def test_needle_128k_layer0():
    """128K: K* of about 400 blocks per head, so the rank check sorts."""
    res, rep = full_layer("needle_128k", 0)
    assert rep["kstar"].max() > 512


@pytest.mark.parametrize("name", ["llama_8k", "llama_32k", "needle_64k", "needle_128k"])
def test_last_layer(name):
    """Layer 31 of each LLaMA-shaped workload (other seeds, positions and
    outlier channels than layer 0)."""
    full_layer(name, 31)


@pytest.mark.parametrize("case", ["all", "default"])
def test_context_above_2048_blocks(case):
    """2100 full blocks and an unfinished one: the selection keeps its
    per-block arrays in global memory (above 2048 blocks) and, with every
    block promoted, the rank check counts pairs in global memory (K* above
    2048)."""
    k, v, q, sm = micro(2100, T=2100 * 64 + 17, Hq=4, Hkv=1, d=64,
                        kind="flat" if case == "all" else "peaked")
    th = oracle.default_thresholds(sm, **(dict(tau_cov=1.0, rank_tol=1.0) if case == "all" else {}))
    res, rep = both(k, v, q, th)
    if case == "all":
        assert np.all(rep["kstar"] == 2100)
        assert np.all(rep["n_discordant"] > 0)


# -- the dense comparator and error paths ---------------------------------------

def to_blocks(k, v):
    """[B][T][Hkv][d] -> block layout [B][Hkv][T/64][...] (K chunk-interleaved,
    V channel-major)."""
    B, T, Hkv, d = k.shape
    kb = k.reshape(B, T // 64, 64, Hkv, d // 8, 8).transpose(0, 3, 1, 4, 2, 5).copy()
    vb = v.reshape(B, T // 64, 64, Hkv, d).transpose(0, 3, 1, 4, 2).copy()
    return kb, vb


def test_dense_comparator_matches_exact_attention():
    import certified_quantized_kv_amd as ckv
    k, v, q, sm = micro(77, T=2048, Hq=8, Hkv=2, d=128, B=2, kind="outliers")
    kb, vb = to_blocks(k, v)
    c = ckv.Cache(1, 2, 8, 2, 128, 2048)
    kt = torch.from_numpy(kb.view(np.float16)).cuda()
    vt = torch.from_numpy(vb.view(np.float16)).cuda()
    qt = torch.from_numpy(q.view(np.float16)).cuda()
    out = c.dense_decode_attention(kt, vt, 2048, qt, sm).cpu().numpy()
    for n in range(2):
        for h in range(8):
            ref = oracle.dense_head(k[n], v[n], q[n, h], h // 4, sm)
            assert np.all(np.abs(out[n, h] - ref) <= ATOL + RTOL * np.abs(ref))
    c.close()


def test_error_paths():
    import certified_quantized_kv_amd as ckv
    c = ckv.Cache(2, 2, 8, 2, 64, 256)
    q = torch.zeros((1, 8, 64), dtype=torch.float16, device="cuda")
    th = oracle.default_thresholds(0.125)
    with pytest.raises(ckv.CkvError) as e:
        c.certified_decode_attention(0, q, th)
    assert e.value.name == "CKV_ESTATE"
    k = np.zeros((200, 2, 64), np.uint16)
    c.append_kv(0, 0, k, k)
    with pytest.raises(ckv.CkvError) as e:
        c.append_kv(0, 0, k, k)
    assert e.value.name == "CKV_ERANGE"
    assert c.seq_length(0, 0) == 200
    with pytest.raises(ckv.CkvError) as e:
        c.certified_decode_attention(5, q, th)
    assert e.value.name == "CKV_EINVAL"
    with pytest.raises(ckv.CkvError) as e:
        c.certified_decode_attention(0, q, dict(th, tau_cov=-0.5))
    assert e.value.name == "CKV_EINVAL"
    out, rep = c.certified_decode_attention(0, q, th)   # all-zero K, V, q: defined
    assert np.all(out.cpu().numpy() == 0)
    c.reset_sequence(0)
    assert c.seq_length(0, 0) == 0
    # the batched one-token append: a full sequence rejects the whole call
    tok = np.zeros((2, 2, 64), np.uint16)
    c.append_kv(0, 1, np.zeros((256, 2, 64), np.uint16), np.zeros((256, 2, 64), np.uint16))
    with pytest.raises(ckv.CkvError) as e:
        c.append_token(0, tok, tok)
    assert e.value.name == "CKV_ERANGE"
    assert c.seq_length(0, 0) == 0 and c.seq_length(0, 1) == 256
    with pytest.raises(ckv.CkvError) as e:
        c.append_token(0, np.zeros((3, 2, 64), np.uint16), np.zeros((3, 2, 64), np.uint16))
    assert e.value.name == "CKV_EINVAL"   # batch above max_batch
    c.append_token(0, tok[:1], tok[:1])
    assert c.seq_length(0, 0) == 1
    c.close()
    with pytest.raises(ckv.CkvError) as e:
        ckv.Cache(1, 1, 8, 2, 64, 256, v_bits=5)
    assert e.value.name == "CKV_EINVAL"

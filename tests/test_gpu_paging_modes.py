"""Device-initiated paging (a kernel reading pinned host memory) against the
host-issued copies: identical outputs, reports and step intermediates, and
parity with the oracle, including sequences skipped by rung 4 before paging
(left to the copies) and the dense fallback after the rank check."""
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


def run_both(k, v, q, th, layers=1):
    import certified_quantized_kv_amd as ckv
    B, T, Hkv, d = k.shape
    Hq = q.shape[1]
    outs = []
    for mode in (False, True):
        c = ckv.Cache(layers, B, Hq, Hkv, d, T)
        c.set_device_paging(mode)
        for l in range(layers):
            for n in range(B):
                c.append_kv(l, n, k[n], v[n])
        res = []
        for l in range(layers):
            out, rep = c.certified_decode_attention(l, torch.from_numpy(q.view(np.float16)).cuda(), th)
            res.append((out.cpu().numpy(), rep, c.export_step(B)))
        outs.append(res)
        c.close()
    for l in range(layers):
        (o0, r0, s0), (o1, r1, s1) = outs[0][l], outs[1][l]
        assert np.array_equal(o0, o1), l
        assert np.array_equal(r0, r1), l
        for key in s0:
            if key != "m16fx":   # defined on P blocks only (checked below)
                assert np.array_equal(s0[key], s1[key]), (l, key)
        B, Hq = r0.shape
        G = Hq // k.shape[2]
        for n in range(B):
            if s0["seq_flags"][n] & 1:   # rung 4 before paging: no FP16-side masses
                continue
            for h in range(Hq):
                sel = s0["sel"][n, h // G, :k.shape[1] // 64]
                inP = ((sel >> (h % G)) & 1).astype(bool)
                assert np.array_equal(s0["m16fx"][n, h, :len(sel)][inP], s1["m16fx"][n, h, :len(sel)][inP]), (l, n, h)
    return outs[1][0]


@pytest.mark.parametrize("case", [dict(), dict(v_cap_blocks=1), dict(rank_tol=-1.0, f_layer=1.0),
                                  dict(rank_tol=-1.0, f_layer=0.5), dict(tau_cov=1.0, v_tol=0.0, k_tol=1.0)])
def test_device_paging_tiny(case):
    L = datagen.make_layer("tiny_1k", 0, T=1000)
    th = oracle.default_thresholds(L.sm, **case)
    out, rep, _ = run_both(L.k, L.v, L.q, th, layers=2)
    res = oracle.certified_decode(L.k, L.v, L.q, th)
    for f in ("kstar", "n_v_promoted", "rung_mask", "e_key", "e_val", "n_discordant"):
        assert np.array_equal(rep[f], res.report[f]), f
    assert np.all(np.abs(out - res.out) <= ATOL + RTOL * np.abs(res.out))


def test_device_paging_batch_d128():
    rng = np.random.default_rng(11)
    B, T, Hq, Hkv, d = 3, 1500, 16, 4, 128
    k = np.asarray(rng.standard_normal((B, T, Hkv, d)), np.float16).view(np.uint16)
    v = np.asarray(rng.standard_normal((B, T, Hkv, d)), np.float16).view(np.uint16)
    q = np.asarray(rng.standard_normal((B, Hq, d)) / np.sqrt(d), np.float16).view(np.uint16)
    th = oracle.default_thresholds(1.0)
    out, rep, _ = run_both(k, v, q, th)
    res = oracle.certified_decode(k, v, q, th)
    assert np.all(np.abs(out - res.out) <= ATOL + RTOL * np.abs(res.out))
    for f in ("kstar", "n_v_promoted", "rung_mask"):
        assert np.array_equal(rep[f], res.report[f]), f


def test_device_paging_llama_8k():
    L = datagen.make_layer("llama_8k", 0)
    th = oracle.default_thresholds(L.sm)
    out, rep, _ = run_both(L.k, L.v, L.q, th)
    res = oracle.certified_decode(L.k, L.v, L.q, th)
    assert np.all(np.abs(out - res.out) <= ATOL + RTOL * np.abs(res.out))
    for f in ("kstar", "n_v_promoted", "rung_mask", "e_key", "e_val"):
        assert np.array_equal(rep[f], res.report[f]), f


def test_device_paging_batch_with_some_sequences_at_rung4_before_paging():
    """The gather starts from the device's own skip flags (written by the
    worklist kernel, before the host reads the selection): sequences 1 and 3
    go to rung 4 before paging (left to the host's copies), sequences 0 and
    2 are certified and paged by the device; identical to host copies and to
    the oracle, two layers in a row."""
    rng = np.random.default_rng(77)
    B, T, Hq, Hkv, d = 4, 1280, 8, 4, 64
    k = rng.standard_normal((B, T, Hkv, d))
    v = rng.standard_normal((B, T, Hkv, d))
    q = rng.standard_normal((B, Hq, d))
    v[0] *= 0.01
    v[2] *= 0.01
    q[1] *= 0.02
    q[3] *= 0.02
    k, v, q = (np.asarray(x, np.float16).view(np.uint16) for x in (k, v, q))
    th = oracle.default_thresholds(1 / np.sqrt(d), v_cap_blocks=2)
    out, rep, step = run_both(k, v, q, th, layers=2)
    res = oracle.certified_decode(k, v, q, th)
    assert list(res.trace["seq_flags"] & 1) == [0, 1, 0, 1]
    assert list(step["seq_flags"] & 1) == [0, 1, 0, 1]
    for f in ("kstar", "n_v_promoted", "rung_max", "rung_mask", "e_key", "e_val", "n_discordant"):
        assert np.array_equal(rep[f], res.report[f]), f
    assert np.all(np.abs(out - res.out) <= ATOL + RTOL * np.abs(res.out))


@pytest.mark.parametrize("name,layer", [("stress_32k", 0), ("stress_32k", 1), ("stress_32k", 2),
                                        ("stress_32k", 3), ("needle_128k", 0)])
def test_device_paging_full_size(name, layer):
    """Full-size layers, device paging against host copies, bit for bit
    (outputs, reports, step intermediates): the stress layers bring every
    rung (the dense fallback pages whole kv groups after the rank check,
    layer 1 sends its sequence to rung 4), the 128K layer gathers lists of
    up to ~2000 blocks per kv head.  The host-copy side is checked against
    the oracle at full size in test_gpu_parity.py."""
    print(f"case device paging {name} layer {layer}", flush=True)
    L = datagen.make_layer(name, layer)
    th = oracle.default_thresholds(L.sm)
    out, rep, step = run_both(L.k, L.v, L.q, th)
    assert np.isfinite(out).all()
    assert (rep["rung_max"] >= 0).all()


@pytest.mark.parametrize("name,layer", [("stress_32k", 0), ("stress_32k", 1), ("stress_32k", 2),
                                        ("stress_32k", 3), ("needle_128k", 0)])
def test_fp16_cache_full_size(name, layer):
    """Full-size layers with the device-resident FP16 block cache against a
    cache without it, bit for bit over two steps (the second query is the
    first with its heads rotated, so it selects other blocks and finds part
    of them mirrored already)."""
    import certified_quantized_kv_amd as ckv
    print(f"case fp16 cache {name} layer {layer}", flush=True)
    L = datagen.make_layer(name, layer)
    th = oracle.default_thresholds(L.sm)
    B, T, Hkv, d = L.k.shape
    Hq = L.q.shape[1]
    qs = [L.q, np.roll(L.q, 1, axis=1).copy()]
    res = []
    for use_cache in (False, True):
        c = ckv.Cache(1, B, Hq, Hkv, d, T)
        if use_cache:
            assert c.enable_fp16_cache(1 << 34) == 1
        for n in range(B):
            c.append_kv(0, n, L.k[n], L.v[n])
        steps = []
        for q in qs:
            out, rep = c.certified_decode_attention(0, torch.from_numpy(q.view(np.float16)).cuda(), th)
            steps.append((out.cpu().numpy(), rep))
        res.append(steps)
        c.close()
    for s in range(2):
        assert np.array_equal(res[0][s][0], res[1][s][0]), s
        assert np.array_equal(res[0][s][1], res[1][s][1]), s

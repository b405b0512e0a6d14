"""Staged paging (host threads pack the listed FP16 blocks into pinned
chunks; one copy and one scatter kernel per chunk) against the run copies:
bit-identical outputs, reports and step intermediates, parity with the
oracle on small layers, and a batch whose chunks wrap the ring of pinned
chunks several times in one step."""
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


def run_modes(k, v, q, th, threads, layers=1, v_bits=4, steps=1, lens=None):
    """The same layers decoded with run copies (threads 0) and with staged
    paging for each entry of `threads`; every result is compared with the
    run copies' and the staged lines' profile is returned."""
    import certified_quantized_kv_amd as ckv
    B, T, Hkv, d = k.shape
    Hq = q.shape[1]
    qt = torch.from_numpy(q.view(np.float16)).cuda()
    base, prof = None, []
    for nt in [0] + list(threads):
        c = ckv.Cache(layers, B, Hq, Hkv, d, T, v_bits=v_bits)
        c.set_staged_paging(nt)
        for l in range(layers):
            for n in range(B):
                t = T if lens is None else lens[n]
                c.append_kv(l, n, k[n, :t], v[n, :t])
        c.set_profiling(True)
        res = []
        for _ in range(steps):
            for l in range(layers):
                out, rep = c.certified_decode_attention(l, qt, th)
                res.append((out.cpu().numpy(), rep, c.export_step(B)))
        if nt:
            prof.append(c.profile())
        c.close()
        if base is None:
            base = res
            continue
        for i, ((o0, r0, s0), (o1, r1, s1)) in enumerate(zip(base, res)):
            assert np.array_equal(o0, o1), (nt, i)
            assert np.array_equal(r0, r1), (nt, i)
            for key in s0:
                if key == "m16fx":   # defined on P blocks only
                    continue
                a0, a1 = s0[key], s1[key]
                if lens is None or a0.ndim < 3:
                    assert np.array_equal(a0, a1), (nt, i, key)
                    continue
                # each sequence's own tokens / block slots (the rest undefined)
                np_ = max(-(-t // 64) for t in lens)
                for n, t in enumerate(lens):
                    m = t if a0.shape[2] == 64 * np_ else -(-t // 64)
                    assert np.array_equal(a0[n, :, :m], a1[n, :, :m]), (nt, i, key, n)
    return base[0], prof


@pytest.mark.parametrize("case", [dict(), dict(v_cap_blocks=1), dict(rank_tol=-1.0, f_layer=1.0),
                                  dict(tau_cov=1.0, v_tol=0.0, k_tol=1.0), dict(tau_cov=0.0)])
def test_staged_paging_tiny(case):
    L = datagen.make_layer("tiny_1k", 0, T=1000)
    th = oracle.default_thresholds(L.sm, **case)
    (out, rep, _), _ = run_modes(L.k, L.v, L.q, th, threads=(1, 3), layers=2)
    res = oracle.certified_decode(L.k, L.v, L.q, th)
    for f in ("kstar", "n_v_promoted", "rung_mask", "e_key", "e_val", "n_discordant"):
        assert np.array_equal(rep[f], res.report[f]), f
    assert np.all(np.abs(out - res.out) <= ATOL + RTOL * np.abs(res.out))


@pytest.mark.parametrize("v_bits", [4, 8])
def test_staged_paging_llama_8k(v_bits):
    L = datagen.make_layer("llama_8k", 0)
    th = oracle.default_thresholds(L.sm)
    (out, rep, _), _ = run_modes(L.k, L.v, L.q, th, threads=(8,), v_bits=v_bits)
    res = oracle.certified_decode(L.k, L.v, L.q, th, v_bits=v_bits)
    assert np.all(np.abs(out - res.out) <= ATOL + RTOL * np.abs(res.out))
    for f in ("kstar", "n_v_promoted", "rung_mask", "e_key", "e_val"):
        assert np.array_equal(rep[f], res.report[f]), f


@pytest.mark.parametrize("d", [128, 64])
def test_staged_paging_wraps_the_ring(d):
    """Every key block listed (tau_cov = 1).  d = 128: sequences of 272, 125,
    125 and 93 blocks; the 272-block runs (at least a chunk's 4 MiB) go as
    direct copies, the other 8 x 343 K blocks as chunks of up to 256 blocks.
    d = 64: 125, 125, 125 and 93 blocks, all packed, in chunks of up to 512
    blocks (a full header of block addresses).  Either way more chunks per
    step than the ring's 16 slots, over two steps (the second step's chunks
    reuse slots of the first's)."""
    rng = np.random.default_rng(23)
    B, Hq, Hkv = 4, 32, 8
    lens = [17408, 8000, 8000, 5952] if d == 128 else [8000, 8000, 8000, 5952]
    T = max(lens)
    k = np.asarray(rng.standard_normal((B, T, Hkv, d)), np.float16).view(np.uint16)
    v = np.asarray(rng.standard_normal((B, T, Hkv, d)), np.float16).view(np.uint16)
    q = np.asarray(rng.standard_normal((B, Hq, d)), np.float16).view(np.uint16)
    th = oracle.default_thresholds(float(1 / np.sqrt(d)), tau_cov=1.0, v_tol=0.0)
    _, prof = run_modes(k, v, q, th, threads=(2, 8), steps=2, lens=lens)
    per_chunk = (4 << 20) // (64 * d * 2)
    direct = lens[0] // 64 >= per_chunk
    packed = Hkv * sum(t // 64 for t in (lens[1:] if direct else lens))
    nblk = Hkv * sum(t // 64 for t in lens)
    for p in prof:
        assert p["copies"] >= 2 * (packed // per_chunk + (Hkv if direct else 0)), p["copies"]
        assert p["bytes_paged"] >= 2 * nblk * 64 * d * 2, p["bytes_paged"]


def test_staged_paging_arguments():
    """Bad thread counts are rejected; switching the thread count, or staged
    paging off and on, between steps of one cache leaves every step's
    results unchanged."""
    import certified_quantized_kv_amd as ckv
    L = datagen.make_layer("tiny_1k", 0, T=1000)
    th = oracle.default_thresholds(L.sm, tau_cov=1.0)
    B, T, Hkv, d = L.k.shape
    c = ckv.Cache(1, B, L.q.shape[1], Hkv, d, T)
    for bad in (-1, 65):
        with pytest.raises(ckv.CkvError) as e:
            c.set_staged_paging(bad)
        assert e.value.status == 1
    for n in range(B):
        c.append_kv(0, n, L.k[n], L.v[n])
    q = torch.from_numpy(L.q.view(np.float16)).cuda()
    res = []
    for nt in (4, 2, 0, 3, 0, 1):
        c.set_staged_paging(nt)
        out, rep = c.certified_decode_attention(0, q, th)
        res.append((out.cpu().numpy(), rep))
    for o, r in res[1:]:
        assert np.array_equal(o, res[0][0])
        assert np.array_equal(r, res[0][1])
    c.close()

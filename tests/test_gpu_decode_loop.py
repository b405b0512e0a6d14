"""Steady-state decode loop: one token appended to every sequence of every
layer per step, then that layer's certified step, compared with the oracle on
each sequence's current prefix.

Each step crosses the unfinished-block path (the trailing block stays FP16 and
exact); every 64th token completes a block, which is quantized at that append
and is bit-exact against the oracle's codes from then on.
"""
import numpy as np
import pytest

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


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 2, 64), (8, 2, 128)])
def test_decode_loop_one_token_per_step(Hq, Hkv, d):
    import certified_quantized_kv_amd as ckv
    L, B, steps = 2, 2, 70
    T0 = [60, 125]                      # start inside a block; both cross block ends
    Tmax = max(T0) + steps
    rng = np.random.default_rng(2024 + d)
    k = f16(rng.standard_normal((L, B, Tmax, Hkv, d)))
    v = f16(rng.standard_normal((L, B, Tmax, Hkv, d)))
    k[1, :, :, :, :4] = f16(10 * rng.standard_normal((B, Tmax, Hkv, 4)))   # outlier channels, layer 1
    sm = float(1 / np.sqrt(d))
    th = oracle.default_thresholds(sm)
    c = ckv.Cache(L, B, Hq, Hkv, d, Tmax)
    for l in range(L):
        for n in range(B):
            c.append_kv(l, n, k[l, n, :T0[n]], v[l, n, :T0[n]])
    for s in range(steps):
        for l in range(L):
            for n in range(B):
                t = T0[n] + s
                tok_k = torch.from_numpy(k[l, n, t:t + 1].view(np.float16)).cuda()
                tok_v = torch.from_numpy(v[l, n, t:t + 1].view(np.float16)).cuda()
                if (s + n) % 2:            # device and host appends alternate
                    c.append_kv(l, n, tok_k, tok_v)
                else:
                    c.append_kv(l, n, k[l, n, t:t + 1], v[l, n, t:t + 1])
            q = f16(rng.standard_normal((B, Hq, d)))
            out, rep = c.certified_decode_attention(l, torch.from_numpy(q.view(np.float16)).cuda(), th)
            out = out.cpu().numpy()
            for n in range(B):
                T = T0[n] + s + 1
                assert c.seq_length(l, n) == T
                res = oracle.certified_decode(k[l, n:n + 1, :T], v[l, n:n + 1, :T], q[n:n + 1], th)
                ctx = (s, l, n, T)
                for f in ("kstar", "n_v_promoted", "rung_mask", "rung_max", "rank_ok", "n_discordant",
                          "e_key", "e_val", "tv_bound", "tau_final"):
                    assert np.array_equal(rep[n][f], res.report[0][f]), (ctx, f)
                ref = res.out[0]
                assert np.all(np.abs(out[n] - ref) <= ATOL + RTOL * np.abs(ref)), \
                    (ctx, np.abs(out[n] - ref).max())
                if T % 64 == 0:            # the block just completed: its codes
                    b = T // 64 - 1
                    tr = res.trace
                    for g in range(Hkv):
                        e = c.export_block(l, n, g, b)
                        assert np.array_equal(e["k_code"], tr["k_code"][0, g, b]), ctx
                        assert np.array_equal(e["v_code"], tr["v_code"][0, g, b]), ctx
                        assert np.array_equal(e["k_s"], tr["k_s"][0, g, b]), ctx
                        assert np.array_equal(e["v_s"], tr["v_s"][0, g, b]), ctx
                        assert e["eta"][0] == tr["eta"][0, g, b], ctx
    c.close()


def test_fp16_cache_same_results_fewer_copies():
    """The device FP16 block cache: the same outputs and reports as paging
    every step, fewer bytes copied from tier 2; a reset sequence's mirrored
    blocks are not reused for its new contents."""
    import certified_quantized_kv_amd as ckv
    L, B, Hq, Hkv, d, T0, steps = 2, 2, 8, 2, 128, 190, 6
    Tmax = T0 + steps + 200
    rng = np.random.default_rng(7)
    k = f16(rng.standard_normal((L, B, Tmax, Hkv, d)))
    v = f16(rng.standard_normal((L, B, Tmax, Hkv, d)))
    th = oracle.default_thresholds(float(1 / np.sqrt(d)), tau_cov=1.0)   # every block in P
    caches = [ckv.Cache(L, B, Hq, Hkv, d, Tmax) for _ in range(2)]
    assert caches[1].enable_fp16_cache(1 << 34) == L
    for c in caches:
        for l in range(L):
            for n in range(B):
                c.append_kv(l, n, k[l, n, :T0], v[l, n, :T0])
        c.set_profiling(True)
    for s in range(steps):
        for l in range(L):
            q = torch.from_numpy(f16(rng.standard_normal((B, Hq, d))).view(np.float16)).cuda()
            res = []
            for c in caches:
                for n in range(B):
                    t = T0 + s
                    c.append_kv(l, n, k[l, n, t:t + 1], v[l, n, t:t + 1])
                out, rep = c.certified_decode_attention(l, q, th)
                res.append((out.cpu().numpy(), rep))
            assert np.array_equal(res[0][0], res[1][0]), (s, l)
            assert np.array_equal(res[0][1], res[1][1]), (s, l)
    p0, p1 = caches[0].profile(), caches[1].profile()
    # every step pages all complete blocks without the cache; with it, each
    # block once (6 steps per layer here: at least 3x fewer bytes)
    assert 0 < p1["bytes_paged"] and 3 * p1["bytes_paged"] <= p0["bytes_paged"], \
        (p0["bytes_paged"], p1["bytes_paged"])
    # a reset sequence gets new contents: the mirror must not serve the old ones
    c = caches[1]
    c.reset_sequence(1)
    for l in range(L):
        c.append_kv(l, 1, k[l, 1, 200:200 + T0][::-1].copy(), v[l, 1, 200:200 + T0][::-1].copy())
    q = f16(rng.standard_normal((B, Hq, d)))
    out, rep = c.certified_decode_attention(0, torch.from_numpy(q.view(np.float16)).cuda(), th)
    kk = k[0, 1:2, 200:200 + T0][:, ::-1].copy()
    vv = v[0, 1:2, 200:200 + T0][:, ::-1].copy()
    ref = oracle.certified_decode(kk, vv, q[1:2], th)
    o = out.cpu().numpy()[1]
    assert np.all(np.abs(o - ref.out[0]) <= ATOL + RTOL * np.abs(ref.out[0]))
    for f in ("kstar", "n_v_promoted", "rung_mask", "e_key", "e_val"):
        assert np.array_equal(rep[1][f], ref.report[0][f]), f
    for c in caches:
        c.close()

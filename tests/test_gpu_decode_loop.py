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


@pytest.mark.parametrize("batched,staged", [(False, 0), (True, 0), (True, 4)])
def test_fp16_cache_same_results_fewer_copies(batched, staged):
    """The device FP16 block cache: the same outputs and reports as paging
    every step, fewer bytes copied from tier 2; a reset sequence's mirrored
    blocks are not reused for its new contents.  batched: the cached cache
    takes its decode tokens through the one-token append (a block completes
    at step 2 while its layer is mirrored).  staged: both caches page with
    staged paging on that many threads."""
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
        c.set_staged_paging(staged)
        for l in range(L):
            for n in range(B):
                c.append_kv(l, n, k[l, n, :T0], v[l, n, :T0])
        c.set_profiling(True)
    for s in range(steps):
        for l in range(L):
            q = torch.from_numpy(f16(rng.standard_normal((B, Hq, d))).view(np.float16)).cuda()
            res = []
            for ci, c in enumerate(caches):
                t = T0 + s
                if batched and ci == 1:
                    c.append_token(l, k[l, :, t].copy(), v[l, :, t].copy())
                else:
                    for n in range(B):
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


@pytest.mark.parametrize("v_bits", [4, 8])
def test_append_token_matches_per_sequence_appends(v_bits):
    """The batched one-token append against ckv_append_kv of the same tokens
    one sequence at a time: identical tier 1 (codes, scales, eta of every
    completed block), identical certified outputs and reports, and tier 2
    read back through a dense-fallback step (rung 4 on every head) equal to
    exact attention.  Sequences start empty, inside a block and at a block
    end, and cross block ends."""
    import certified_quantized_kv_amd as ckv
    Hq, Hkv, d, B, steps = 8, 2, 128, 3, 140
    T0 = [0, 37, 64]
    Tmax = max(T0) + steps
    rng = np.random.default_rng(77 + v_bits)
    k = f16(rng.standard_normal((B, Tmax, Hkv, d)))
    v = f16(rng.standard_normal((B, Tmax, Hkv, d)))
    sm = float(1 / np.sqrt(d))
    th = oracle.default_thresholds(sm)
    a = ckv.Cache(1, B, Hq, Hkv, d, Tmax, v_bits=v_bits)
    b = ckv.Cache(1, B, Hq, Hkv, d, Tmax, v_bits=v_bits)
    for n in range(B):
        if T0[n]:
            a.append_kv(0, n, k[n, :T0[n]], v[n, :T0[n]])
            b.append_kv(0, n, k[n, :T0[n]], v[n, :T0[n]])
    for s in range(steps):
        tk = np.stack([k[n, T0[n] + s] for n in range(B)])
        tv = np.stack([v[n, T0[n] + s] for n in range(B)])
        if s % 2:   # device and host sources alternate
            a.append_token(0, torch.from_numpy(tk.view(np.float16)).cuda(),
                           torch.from_numpy(tv.view(np.float16)).cuda())
        else:
            a.append_token(0, tk, tv)
        for n in range(B):
            b.append_kv(0, n, k[n, T0[n] + s:T0[n] + s + 1], v[n, T0[n] + s:T0[n] + s + 1])
        if s % 35 == 34 or s == steps - 1:
            for n in range(B):
                assert a.seq_length(0, n) == b.seq_length(0, n) == T0[n] + s + 1
                for g in range(Hkv):
                    for blk in range((T0[n] + s + 1) // 64):
                        ea, eb = a.export_block(0, n, g, blk), b.export_block(0, n, g, blk)
                        for f in ea:
                            assert np.array_equal(ea[f], eb[f]), (s, n, g, blk, f)
            q = torch.from_numpy(f16(rng.standard_normal((B, Hq, d))).view(np.float16)).cuda()
            oa, ra = a.certified_decode_attention(0, q, th)
            ob, rb = b.certified_decode_attention(0, q, th)
            assert torch.equal(oa, ob) and np.array_equal(ra, rb), s
    # tier 2: every head falls back (rank_tol < 0, f_layer = 0): the output is
    # exact attention over the FP16 blocks paged from tier 2 and the device
    # copy of the unfinished block
    thd = oracle.default_thresholds(sm, rank_tol=-1.0, f_layer=0.0)
    q = f16(rng.standard_normal((B, Hq, d)))
    out, rep = a.certified_decode_attention(0, torch.from_numpy(q.view(np.float16)).cuda(), thd)
    out = out.cpu().numpy()
    assert np.all(rep["rung_max"] == 4)
    for n in range(B):
        T = T0[n] + steps
        res = oracle.certified_decode(k[n:n + 1, :T], v[n:n + 1, :T], q[n:n + 1], thd, v_bits=v_bits)
        ref = res.trace["o_dense"][0]
        assert np.all(np.abs(out[n] - ref) <= ATOL + RTOL * np.abs(ref)), n
    a.close()
    b.close()

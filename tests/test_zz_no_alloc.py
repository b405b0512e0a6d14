"""The allocation-free dense entry point (ckv_dense_decode_attention_noalloc)
against the cached one (ckv_dense_decode_attention) and against exact
attention, through the C ABI.

Both compute exact dense decode attention over FP16 blocks, the fallback of
"Runtime-Certified Bounded-Error Quantized Attention" (technical summary,
Methodology 1 and Key contributions: exact O_dense when the bounds cannot be
met) and the dense comparator of its Experimental results.  Outputs within
2e-3 absolute + 1e-2 relative (FP32 accumulation against the oracle's FP64).
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
    import certified_quantized_kv_amd as ckv  # noqa: F401


def f16(x):
    return np.asarray(x, np.float16).view(np.uint16)


def inputs(seed, B, T, Hq, Hkv, d):
    rng = np.random.default_rng(seed)
    k = f16(rng.standard_normal((B, T, Hkv, d), dtype=np.float32))
    v = f16(rng.standard_normal((B, T, Hkv, d), dtype=np.float32))
    q = f16(rng.standard_normal((B, Hq, d), dtype=np.float32))
    # block layout: K [head_dim/8][64][8], V [head_dim][64] per block
    kb = k.reshape(B, T // 64, 64, Hkv, d // 8, 8).transpose(0, 3, 1, 4, 2, 5).copy()
    vb = v.reshape(B, T // 64, 64, Hkv, d).transpose(0, 3, 1, 4, 2).copy()
    dev = lambda a: torch.from_numpy(a.view(np.float16)).cuda()  # noqa: E731
    return k, v, q, dev(kb), dev(vb), dev(q), float(1 / np.sqrt(d))


def noalloc(kt, vt, T, qt, sm, Hkv):
    from certified_quantized_kv_amd import binding
    B, Hq, d = qt.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    binding.dense_decode_attention_noalloc(kt, vt, T, qt, sm, Hkv, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def check_exact(out, k, v, q, sm, heads):
    Hkv, Hq = k.shape[2], q.shape[1]
    for n, h in heads:
        ref = oracle.dense_head(k[n], v[n], q[n, h], h // (Hq // Hkv), sm)
        assert np.all(np.abs(out[n, h] - ref) <= ATOL + RTOL * np.abs(ref)), (n, h)


def test_noalloc_matches_the_cached_entry_point_on_consecutive_calls():
    """Two calls in a row (the second smaller), then a third of another head
    shape: each against the cached entry point and exact attention."""
    import certified_quantized_kv_amd as ckv
    for i, (B, T, Hq, Hkv, d) in enumerate([(2, 8192, 32, 8, 128), (1, 2048, 32, 8, 128),
                                            (3, 1024, 8, 1, 64)]):
        print(f"case call {i} B={B} T={T} Hq={Hq} Hkv={Hkv} d={d}", flush=True)
        k, v, q, kt, vt, qt, sm = inputs(10 + i, B, T, Hq, Hkv, d)
        got = noalloc(kt, vt, T, qt, sm, Hkv)
        with ckv.Cache(1, B, Hq, Hkv, d, T) as c:
            want = c.dense_decode_attention(kt, vt, T, qt, sm)
            torch.cuda.synchronize()
            want = want.cpu().numpy().astype(np.float64)
        # the same splits and kernels: the same bits
        assert np.array_equal(got, want), i
        check_exact(got, k, v, q, sm, [(n, h) for n in range(B) for h in range(Hq)])


def test_noalloc_longer_splits_when_the_scratch_is_short():
    """8 sequences x 64 q heads at 128K tokens (head_dim 64): the cached
    entry point's 32 splits per head would need more than the 4 MiB scratch,
    so the allocation-free pass takes fewer, longer splits."""
    B, T, Hq, Hkv, d = 8, 131072, 64, 8, 64
    print(f"case longer splits B={B} T={T} Hq={Hq}", flush=True)
    assert B * Hq * 32 * (d + 2) * 4 > 4 << 20
    k, v, q, kt, vt, qt, sm = inputs(7, B, T, Hq, Hkv, d)
    got = noalloc(kt, vt, T, qt, sm, Hkv)
    check_exact(got, k, v, q, sm, [(0, 0), (3, 17), (7, 63)])
    # a small call right after still gives the cached entry point's bits
    import certified_quantized_kv_amd as ckv
    k, v, q, kt, vt, qt, sm = inputs(8, 1, 1024, 8, 2, 64)
    got = noalloc(kt, vt, 1024, qt, sm, 2)
    with ckv.Cache(1, 1, 8, 2, 64, 1024) as c:
        want = c.dense_decode_attention(kt, vt, 1024, qt, sm)
        torch.cuda.synchronize()
    assert np.array_equal(got, want.cpu().numpy().astype(np.float64))


def test_noalloc_rejects_shapes_beyond_the_scratch_and_bad_arguments():
    from certified_quantized_kv_amd import binding
    import certified_quantized_kv_amd as ckv
    k, v, q, kt, vt, qt, sm = inputs(3, 1, 64, 8, 2, 64)
    out = torch.empty((1, 8, 64), dtype=torch.float32, device="cuda")
    # batch x q heads whose single split per head exceeds 4 MiB
    big_q = torch.zeros((256, 64, 128), dtype=torch.float16, device="cuda")
    big_out = torch.empty((256, 64, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(ckv.CkvError) as e:
        binding.dense_decode_attention_noalloc(kt, vt, 64, big_q, sm, 8, big_out)
    assert e.value.name == "CKV_EINVAL" and "scratch" in str(e.value)
    for args in [(kt, vt, 100, qt, sm, 2, out),     # not a multiple of 64
                 (kt, vt, 64, qt, -1.0, 2, out),    # scale
                 (kt, vt, 64, qt, sm, 3, out)]:     # heads not a multiple
        with pytest.raises(ckv.CkvError) as e:
            binding.dense_decode_attention_noalloc(*args)
        assert e.value.name == "CKV_EINVAL"
    # a good call after the rejected ones
    got = noalloc(kt, vt, 64, qt, sm, 2)
    check_exact(got, k, v, q, sm, [(0, h) for h in range(8)])

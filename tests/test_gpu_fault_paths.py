"""Error path of a decode step, forced from the host.

A paging copy is made to report failure (ckv_inject_paging_fault: the copy
is not issued, as if hipMemcpyAsync had failed); no kernel faults.  The step
must return CKV_EHIP with every head at rung_max = -1, and the next step on
the same cache must give the oracle's result: blocks that the failed step
listed for paging were never copied, so the cache must not treat them as
staged (with the device-resident FP16 cache on, those flags persist across
steps).  The guarantee exercised is the deterministic-recovery contribution
of "Runtime-Certified Bounded-Error Quantized Attention" (technical
summary, Key contributions): a step either returns a certified or exact
result, or an error, never a silently wrong output.
"""
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
    import certified_quantized_kv_amd as ckv  # noqa: F401


def check_against_oracle(res, out, rep):
    for f in ("kstar", "n_v_promoted", "rank_ok", "n_discordant", "rung_max", "rung_mask", "e_key",
              "e_val", "tv_bound", "tau_final"):
        assert np.array_equal(rep[f], res.report[f]), f
    out = out.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(out - res.out) <= ATOL + RTOL * np.abs(res.out))


@pytest.mark.parametrize("staged", [True, False])
@pytest.mark.parametrize("fp16_cache", [False, True])
@pytest.mark.parametrize("after", [0, 1])
def test_failed_paging_copy_reports_error_and_next_step_recovers(staged, fp16_cache, after):
    import certified_quantized_kv_amd as ckv
    print(f"case staged={staged} fp16_cache={fp16_cache} after={after}", flush=True)
    L = datagen.make_layer("llama_8k", 2)
    B, T, Hkv, d = L.k.shape
    Hq = L.q.shape[1]
    th = oracle.default_thresholds(L.sm)
    res = oracle.certified_decode(L.k, L.v, L.q, th, trace=False)
    # a second query: with the FP16 cache on, its step needs blocks that the
    # first step did not page
    rng = np.random.default_rng(9)
    q2 = (L.q.view(np.float16).astype(np.float64) + rng.standard_normal(L.q.shape) / np.sqrt(d))
    q2 = q2.astype(np.float16).view(np.uint16)
    res2 = oracle.certified_decode(L.k, L.v, q2, th, trace=False)
    with ckv.Cache(1, B, Hq, Hkv, d, T) as c:
        if not staged:
            c.set_staged_paging(0)
        if fp16_cache:
            assert c.enable_fp16_cache(1 << 40) == 1
        c.append_kv(0, 0, L.k[0], L.v[0])
        qd = torch.from_numpy(L.q.view(np.float16)).cuda()
        q2d = torch.from_numpy(q2.view(np.float16)).cuda()
        # a good step first (with the FP16 cache, some blocks stay staged)
        out, rep = c.certified_decode_attention(0, qd, th)
        check_against_oracle(res, out, rep)
        # the failing step
        c.inject_paging_fault(after)
        with pytest.raises(ckv.CkvError) as e:
            c.certified_decode_attention(0, q2d, th)
        assert e.value.name == "CKV_EHIP"
        assert np.all(e.value.report["rung_max"] == -1)
        torch.cuda.synchronize()
        # the next steps on the same cache are right
        out, rep = c.certified_decode_attention(0, q2d, th)
        check_against_oracle(res2, out, rep)
        out, rep = c.certified_decode_attention(0, qd, th)
        check_against_oracle(res, out, rep)


def test_fault_injection_clears_itself_and_can_be_cancelled():
    import certified_quantized_kv_amd as ckv
    L = datagen.make_layer("tiny_1k", 0)
    B, T, Hkv, d = L.k.shape
    th = oracle.default_thresholds(L.sm)
    res = oracle.certified_decode(L.k, L.v, L.q, th, trace=False)
    with ckv.Cache(1, B, L.q.shape[1], Hkv, d, T) as c:
        c.append_kv(0, 0, L.k[0], L.v[0])
        qd = torch.from_numpy(L.q.view(np.float16)).cuda()
        c.inject_paging_fault(0)
        c.inject_paging_fault(-1)          # cancelled: the step succeeds
        out, rep = c.certified_decode_attention(0, qd, th)
        check_against_oracle(res, out, rep)
        c.inject_paging_fault(0)
        with pytest.raises(ckv.CkvError):
            c.certified_decode_attention(0, qd, th)
        out, rep = c.certified_decode_attention(0, qd, th)   # fired once only
        check_against_oracle(res, out, rep)

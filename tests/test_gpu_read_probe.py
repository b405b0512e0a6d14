"""ckv_read_probe, the streaming-read measurement aid: it reads every wave's
share (a wave whose loaded words fold to the marker value reports its index,
so a wrong offset or a skipped wave shows), and it rejects bad arguments on
the host before any launch."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MARK = 0x9E3779B9


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("kib", [4, 8, 16])
@pytest.mark.parametrize("wave", [0, 5, 127])
def test_each_wave_reads_its_own_share(kib, wave):
    from certified_quantized_kv_amd import binding
    n_waves = 128
    words = np.zeros(n_waves * kib * 256, dtype=np.uint32)
    # one marked word, at a lane and load other than the first, in `wave`'s
    # share: only that wave's fold equals the marker
    words[wave * kib * 256 + (kib - 1) * 256 + 37 * 4 + 2] = MARK
    buf = torch.from_numpy(words.view(np.int32)).to("cuda:0")
    sink = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    binding.read_probe(buf, kib, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == wave


def test_unmarked_buffer_writes_nothing():
    from certified_quantized_kv_amd import binding
    buf = torch.zeros(64 * 2048, dtype=torch.int32, device="cuda:0")
    sink = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    binding.read_probe(buf, 8, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == -1


def test_bad_arguments_are_rejected():
    from certified_quantized_kv_amd import binding
    L = binding.lib()
    buf = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    p, s = ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(sink.data_ptr())
    nb = buf.numel() * 4
    assert L.ckv_read_probe(p, nb, 3, s, None) == 1          # wave_kib
    assert L.ckv_read_probe(p, nb - 1024, 16, s, None) == 1  # not a multiple of 16 KiB
    assert L.ckv_read_probe(p, 0, 8, s, None) == 1
    assert L.ckv_read_probe(None, nb, 8, s, None) == 1
    assert L.ckv_read_probe(p, nb, 8, None, None) == 1
    assert b"null" in L.ckv_last_error()
    assert L.ckv_read_probe(p, nb, 8, s, None) == 0
    torch.cuda.synchronize()

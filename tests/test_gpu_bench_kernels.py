"""The measurement kernels that bench.py relies on: the streaming read that
sets the achievable-bandwidth ceiling must touch every 32-bit word of its
buffer exactly once (the XOR of its per-workgroup checksums is the XOR of
all words; a word read twice or skipped changes it), and the calibration
copy must copy exactly its bytes.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)

import paged_kv_cache_250_amd as pkv  # noqa: E402
from gpu_common import note  # noqa: E402

SIZES = [16, 1008, 1024, 4096 + 48, (1 << 20) + 16 * 37, 64 << 20, (256 << 20) + 1024 * 5 + 32]


@pytest.mark.parametrize("nbytes", SIZES)
def test_stream_read_reads_every_word_once(nbytes):
    note(f"stream_read bytes={nbytes}")
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    # distinct words, so that a word read twice (cancelling) or skipped
    # leaves a different XOR
    words[::7] ^= np.arange(0, words[::7].size, dtype=np.uint32) * np.uint32(2654435761)
    buf = torch.from_numpy(words.view(np.uint8)).cuda()
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    pkv.pkv_bench_stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
    # and a stale or missing word changes it: flip one word in the tail
    words[-1] ^= np.uint32(0x80000001)
    buf[-4:] = torch.from_numpy(words[-1:].view(np.uint8)).cuda()
    sink.zero_()
    pkv.pkv_bench_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == \
        np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("nbytes", [16, 1008, (1 << 20) + 48])
def test_bench_copy_copies_exactly(nbytes):
    note(f"bench_copy bytes={nbytes}")
    rng = np.random.default_rng(nbytes + 1)
    src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    dst = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    pkv.pkv_bench_copy(dst[:nbytes], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert bool((dst[nbytes:] == 0xA5).all())


def test_bench_copy_uploads_pinned_host_memory():
    """The bench's per-step upload: the copy kernel reads a pinned host
    buffer through its device address and writes exactly its bytes, each
    time the host refills the buffer (no stale host bytes)."""
    import ctypes
    import sys

    from conftest import ROOT
    sys.path.insert(0, ROOT)
    import bench

    note("bench_copy from pinned host memory")
    n = 3 * 64 + 64 * 258
    n = -(-n // 4) * 4
    host = torch.empty(n, dtype=torch.int32).pin_memory()
    src = bench.pinned_device_address(host)
    dst = torch.full((n + 16,), -1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rng = np.random.default_rng(11)
    for _ in range(4):
        host.copy_(torch.from_numpy(rng.integers(-2**31, 2**31 - 1, n, dtype=np.int32)))
        pkv._check(pkv._lib.pkv_bench_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src),
                                           ctypes.c_size_t(n * 4), ctypes.c_void_p(stream)))
        torch.cuda.synchronize()
        assert torch.equal(dst[:n].cpu(), host)
        assert bool((dst[n:] == -1).all())

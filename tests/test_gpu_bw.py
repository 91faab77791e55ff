"""The benchmark's read-bandwidth reference kernel (libmla_bw.so) reads
every word of its buffer exactly once: the XOR of everything it writes to
its sink equals the XOR of all words of the buffer, for any grid size."""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("blocks", [1, 3, 64, 4096])
def test_read_reference_reads_every_word_once(blocks):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw = ctypes.CDLL(os.path.join(ROOT, "mla_paged_kv_metadata_amd", "libmla_bw.so"))
    bw.mla_bw_read.restype = ctypes.c_int
    bw.mla_bw_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    rng = np.random.default_rng(blocks)
    words = rng.integers(0, 2**32, size=(32768 // 4) * 37, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    sink = torch.full((blocks * 4,), -1, dtype=torch.int32, device="cuda")
    rc = bw.mla_bw_read(src.data_ptr(), words.nbytes, sink.data_ptr(), blocks,
                        torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)

"""The benchmark's bandwidth references (libstream_ref.so): a plain copy and
a plain read.  Not part of the LoRA library; checked so that the ceilings
the benchmark reports come from kernels that do what they say."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PATH = os.path.join(ROOT, "rank_specialized_amd", "libstream_ref.so")


def _lib():
    if not os.path.exists(PATH):
        pytest.skip("libstream_ref.so not built")
    lib = ctypes.CDLL(PATH)
    lib.stream_ref_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.stream_ref_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.stream_ref_copy.restype = lib.stream_ref_read.restype = ctypes.c_int
    return lib


def test_reference_rejects_bad_arguments_before_any_hip_call():
    """Sizes that are not whole 16-byte elements, missing or misaligned
    pointers: 1, with no launch; a zero size: 0."""
    lib = _lib()
    assert lib.stream_ref_copy(16, 32, 17, None) == 1
    assert lib.stream_ref_copy(None, 32, 16, None) == 1
    assert lib.stream_ref_copy(16, 40, 16, None) == 1
    assert lib.stream_ref_read(16, 8, 64, None) == 1
    assert lib.stream_ref_read(16, 16, None, None) == 1
    assert lib.stream_ref_copy(None, None, 0, None) == 0
    assert lib.stream_ref_read(None, 0, None, None) == 0


@pytest.mark.gpu
def test_reference_copy_is_exact():
    """The copy writes every byte of the source and nothing past it (a
    ragged size: 3 workgroups and a partial one)."""
    import torch
    lib = _lib()
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5)
    n = 16 * (3 * 256 + 77)
    src = torch.from_numpy(rng.integers(0, 256, size=n, dtype=np.uint8)).to(dev)
    dst = torch.full((n + 256,), 0xA5, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.stream_ref_copy(src.data_ptr(), dst.data_ptr(), n, stream) == 0
    assert lib.stream_ref_read(src.data_ptr(), n, sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    out = dst.cpu().numpy()
    assert np.array_equal(out[:n], src.cpu().numpy())
    assert (out[n:] == 0xA5).all()

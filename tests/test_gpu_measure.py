"""The measurement kernels behind bench.py's launch floor and streaming ceiling
(include/pace_measure.h) on the GPU: the stream kernel reads every byte of each workgroup's
slice (its one-word result per workgroup equals the XOR of the slice's 32-bit words, computed
on the host), in the decode's launch shape and in shapes with a ragged tail; the empty kernel
launches.  A ceiling measured with a kernel that skipped bytes would not bound anything."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    import bit_recurrent_state_amd  # noqa: F401  (torch's HIP runtime and libpace first)
    lib = ctypes.CDLL(os.path.join(ROOT, "bit_recurrent_state_amd", "libpace_measure.so"))
    lib.pace_measure_empty.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.pace_measure_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("gx,gy,threads,bytes_per_wg", [
    (32, 64, 128, 11472),      # the decode's grid at B = 64 and its bytes per workgroup (rounded to 16)
    (3, 5, 64, 16 * 1000),     # a tail after the 8-deep loop
    (2, 2, 256, 16),           # one vector per workgroup
    (7, 1, 1024, 16 * 8 * 1024 * 3 + 48),
])
def test_stream_kernel_reads_every_byte(gx, gy, threads, bytes_per_wg):
    print(f"[measure] stream gx={gx} gy={gy} threads={threads} bytes/wg={bytes_per_wg}", flush=True)
    lib = _lib()
    n = gx * gy * bytes_per_wg
    rng = np.random.default_rng(gx * 1000 + gy)
    host = rng.integers(0, 2 ** 32, size=n // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(gx * gy, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.pace_measure_stream(ctypes.c_void_p(src.data_ptr()), bytes_per_wg, gx, gy, threads,
                                 ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream))
    assert rc == 0
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(host.reshape(gx * gy, bytes_per_wg // 4), axis=1)
    assert np.array_equal(got, want)


def test_empty_kernel_launches_in_the_decode_shape():
    lib = _lib()
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.pace_measure_empty(32, 64, 128, ctypes.c_void_p(stream)) == 0
    torch.cuda.synchronize()

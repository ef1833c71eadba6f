"""GPU checks of the calibration kernels behind bench.py's measured peaks
(libpic_calib.so, include/pic_calib.h): each computes what its rate is credited for."""

import ctypes
import os

import numpy as np
import pytest

import position_independent_kv_rope_amd as P  # noqa: F401  (package import path)
from position_independent_kv_rope_amd import build

pytestmark = pytest.mark.gpu


def _lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(build.CALIB_LIB):
        raise RuntimeError("libpic_calib.so is missing; run build() first")
    L = ctypes.CDLL(build.CALIB_LIB)
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.pic_calib_read_sink_words.argtypes = [i64]
    L.pic_calib_read_sink_words.restype = i64
    L.pic_calib_read.argtypes = [p, i64, p, p]
    L.pic_calib_copy.argtypes = [p, p, i64, p]
    L.pic_calib_update.argtypes = [p, i64, p]
    L.pic_calib_mfma.argtypes = [p, p, i32, i32, p]
    L.pic_calib_mfma_flops.argtypes = [i32, i32]
    L.pic_calib_mfma_flops.restype = i64
    return L


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


@pytest.mark.parametrize("n_bytes", [16, 4096 * 16 + 48, 64 << 20])
def test_stream_copy_update_and_read(n_bytes):
    import torch
    L = _lib()
    g = torch.Generator(device="cpu").manual_seed(n_bytes)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_bytes // 4,), dtype=torch.int32, generator=g)
    src = host.cuda()
    dst = torch.zeros_like(src)
    assert L.pic_calib_copy(src.data_ptr(), dst.data_ptr(), n_bytes, _stream()) == 0
    sink = torch.full((int(L.pic_calib_read_sink_words(n_bytes)),), 7, dtype=torch.int32,
                      device="cuda")
    assert L.pic_calib_read(src.data_ptr(), n_bytes, sink.data_ptr(), _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), host)
    assert L.pic_calib_update(dst.data_ptr(), n_bytes, _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), ~host)
    # every 32-bit word of the buffer enters exactly one wave's XOR
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


def test_mfma_loop_computes_its_products():
    # one wave's chain c accumulates A_c (32 x 16) times B_{(c + r) % 4} (16 x 32) for
    # rounds r = 0 .. iters-1, so the sum of all its outputs over the wave is
    # (iters / 4) * sum_k colsum(A_c)[k] * rowsum(B_0 + B_1 + B_2 + B_3)[k], whichever
    # lane holds which element (A and B fragments share one k order)
    import torch
    L = _lib()
    n_wg, iters = 8, 64
    g = torch.Generator(device="cpu").manual_seed(3)
    ops = (torch.rand(8 * 64 * 8, generator=g) - 0.5).to(torch.bfloat16)
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    assert L.pic_calib_mfma(ops.cuda().data_ptr(), sink.data_ptr(), n_wg, iters, _stream()) == 0
    torch.cuda.synchronize()
    frag = ops.to(torch.float64).numpy().reshape(8, 64, 8)  # [fragment][lane][8 values]

    def kmat(f):  # [16 k][32 rows or columns]: lane l holds k = 8 * (l // 32) + e, index l % 32
        m = np.zeros((16, 32))
        for lane in range(64):
            m[8 * (lane // 32):8 * (lane // 32) + 8, lane % 32] = f[lane]
        return m

    a = [kmat(frag[c]) for c in range(4)]          # A_c^T: [k][row]
    b = sum(kmat(frag[4 + c]) for c in range(4))   # (B_0 + ... + B_3): [k][column]
    want = (iters // 4) * sum(float(np.dot(a[c].sum(axis=1), b.sum(axis=1))) for c in range(4))
    per_wave = sink.cpu().to(torch.float64).numpy().reshape(n_wg * 4, 64).sum(axis=1)
    assert np.allclose(per_wave, want, rtol=1e-4, atol=1e-3), (per_wave[:4], want)
    assert L.pic_calib_mfma_flops(n_wg, iters) == n_wg * 4 * iters * 4 * 32768

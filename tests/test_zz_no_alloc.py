"""The allocation-free prefill entry point (q4k_f16_gemm_f32x_noalloc):
through the C ABI it must give exactly what q4k_f16_gemm_f32x gives with a
caller scratch (the same kernels on the same fp16 activations), on two calls
in a row, the second smaller (the static array keeps the first call's
activations beyond the second's), and refuse m*k beyond its 4 Mi halves
before any HIP call."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_quantized_decode_q4_amd import q4k  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4k.load_library()
    yield


def _pair(lib, m, n, k, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    w16 = (torch.randn((n, k), device="cuda", generator=g) * 0.05).to(torch.float16)
    x = torch.randn((m, k), device="cuda", generator=g)
    xh = torch.empty((m, k), dtype=torch.float16, device="cuda")
    y_ref = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    rc = lib.q4k_f16_gemm_f32x(w16.data_ptr(), x.data_ptr(), xh.data_ptr(), y_ref.data_ptr(),
                               m, n, k, s)
    assert rc == 0, rc
    rc = lib.q4k_f16_gemm_f32x_noalloc(w16.data_ptr(), x.data_ptr(), y.data_ptr(), m, n, k, s)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return y.cpu().numpy(), y_ref.cpu().numpy()


def test_noalloc_matches_the_scratch_entry_point_twice():
    lib = q4k.load_library()
    for m, n, k, seed in ((300, 500, 1024, 1), (64, 200, 256, 2)):
        print("noalloc m=%d n=%d k=%d" % (m, n, k), flush=True)
        y, y_ref = _pair(lib, m, n, k, seed)
        assert np.isfinite(y_ref).all()
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32))


def test_noalloc_refuses_beyond_its_scratch():
    lib = q4k.load_library()
    a = 0x100000
    assert lib.q4k_f16_gemm_f32x_noalloc(a, a, a, 4097, 64, 1024, None) == q4k.Q4K_ERR_UNSUPPORTED
    assert lib.q4k_f16_gemm_f32x_noalloc(a, None, a, 8, 64, 64, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_f16_gemm_f32x_noalloc(a, a, a, 8, 64, 96, None) == q4k.Q4K_ERR_UNSUPPORTED

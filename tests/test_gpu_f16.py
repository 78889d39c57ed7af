"""GPU parity of the prefill step beside the decode path: the fp16 mirror
(q4k_mirror_f16, q6k_mirror_f16), the activation convert (q4k_f16_cvt) and
the fp16 GEMM on the matrix cores (q4k_f16_gemm, q4k_f16_gemm_f32x)
(memra-engine 0.83.1, src/f16_ffi.rs: `memra_q4_K_dequant_f16`,
`memra_q6_K_dequant_f16`, `memra_f16_cvt`, `memra_f16_pp_gemm`).

The mirror and the convert are integer work decided in f32 on both sides:
bit-exact against the oracle (NaN compared as NaN).  The GEMM is held to
|y - y_ref| <= k * 2^-23 * sum|w16||x16| per output, y_ref the oracle's
exact dot product of the fp16 operands (oracle.f16_gemm): products of two
binary16 values are exact in f32 and an f32 sum of k terms in any order errs
by at most (k - 1) 2^-24 of the sum of magnitudes.  Shapes span several
tiles with ragged m and n; the full prefill shape is checked on sampled
blocks of outputs.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_quantized_decode_q4_amd import q4k, synth  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4k.load_library()
    yield


def _say(msg):
    print(msg, flush=True)


def _same_bits_or_nan(a16, b16):
    a = np.asarray(a16, np.uint16)
    b = np.asarray(b16, np.uint16)
    nan_a = ((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)
    nan_b = ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return np.array_equal(nan_a, nan_b) and np.array_equal(a[~nan_a], b[~nan_b])


def test_q4k_mirror_bit_exact(oracle_mod):
    for n, k, seed in ((37, 2048, 1), (256, 1024, 2)):
        f = synth.draw_fields(np.random.default_rng(4000 + seed), n, k // 256)
        f.d_bits[0, 0] = 0x7800          # weights beyond the fp16 range -> inf
        f.d_bits[1, 1] = 0x7E00          # NaN d
        f.d_bits[2, 0] = 0x0001          # subnormal d
        w = synth.pack(f)
        _say("q4k mirror n=%d k=%d" % (n, k))
        w_d = torch.from_numpy(w).cuda()
        out = torch.zeros((n, k), dtype=torch.int16, device="cuda")
        q4k.q4k_mirror_f16(w_d, out, n, k)
        torch.cuda.synchronize()
        assert _same_bits_or_nan(out.cpu().numpy().view(np.uint16),
                                 oracle_mod.mirror_f16(w, 4, n, k))


def test_q6k_mirror_bit_exact(oracle_mod):
    for n, k, stride in ((37, 2048, 0), (64, 1024, 896)):
        f = synth.draw_q6k_fields(np.random.default_rng(4100 + n), n, k // 256)
        f.d_bits[0, 0] = 0x7BFF          # largest d: some weights beyond the fp16 range
        w = synth.pack_q6k(f, stride)
        _say("q6k mirror n=%d k=%d stride=%d" % (n, k, stride))
        w_d = torch.from_numpy(w).cuda()
        out = torch.zeros((n, k), dtype=torch.int16, device="cuda")
        q4k.q6k_mirror_f16(w_d, out, n, k, stride)
        torch.cuda.synchronize()
        assert _same_bits_or_nan(out.cpu().numpy().view(np.uint16),
                                 oracle_mod.mirror_f16(w, 6, n, k, stride))


def test_f16_cvt_bit_exact(oracle_mod):
    rng = np.random.default_rng(4201)
    for count in (1, 7, 4096, 100003):
        x = (rng.standard_normal(count) * np.exp2(rng.integers(-30, 20, size=count))).astype(np.float32)
        x[: min(count, 6)] = [0.0, -0.0, 65504.0, 65520.0, np.inf, -1e-8][: min(count, 6)]
        _say("f16 cvt count=%d" % count)
        x_d = torch.from_numpy(x).cuda()
        out = torch.zeros(count, dtype=torch.int16, device="cuda")
        q4k.q4k_f16_cvt(x_d, out, count)
        torch.cuda.synchronize()
        assert _same_bits_or_nan(out.cpu().numpy().view(np.uint16), oracle_mod.f16_cvt(x))


def _gemm_gpu(w16, x16, m, n, k):
    w_d = torch.from_numpy(np.ascontiguousarray(w16).view(np.int16)).cuda()
    x_d = torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).cuda()
    y_d = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    q4k.q4k_f16_gemm(w_d, x_d, y_d, m, n, k)
    torch.cuda.synchronize()
    return y_d.cpu().numpy()


def _check_gemm(y, y_ref, bound, k, what):
    err = np.abs(y.astype(np.float64) - y_ref)
    tol = k * 2.0 ** -23 * bound
    bad = ~(err <= tol)
    assert not bad.any(), "%s: %d outputs outside k 2^-23 sum|w||x|, first %s" % (
        what, int(bad.sum()), tuple(np.argwhere(bad)[0]))
    worst = float((err / np.maximum(tol, 1e-300)).max())
    _say("  %s: worst |err| / tolerance %.3g" % (what, worst))


@pytest.mark.parametrize("m,n,k", [(1, 1, 64), (5, 7, 64), (128, 128, 128), (130, 300, 256),
                                   (257, 129, 512), (64, 1000, 1024)])
def test_f16_gemm_shapes(oracle_mod, m, n, k):
    rng = np.random.default_rng(4300 + m + n + k)
    w16 = oracle_mod.f16_cvt((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    x16 = oracle_mod.f16_cvt(rng.standard_normal((m, k)).astype(np.float32))
    _say("f16 gemm m=%d n=%d k=%d" % (m, n, k))
    y = _gemm_gpu(w16, x16, m, n, k)
    y_ref, bound = oracle_mod.f16_gemm(w16, x16)
    _check_gemm(y, y_ref, bound, k, "m=%d n=%d k=%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k,tile", [(512, 14336, 128, "128 x 128"), (512, 6144, 128, "64 x 128"),
                                        (500, 4100, 192, "64 x 128"), (500, 3000, 320, "64 x 64")])
def test_f16_gemm_tile_variants(oracle_mod, m, n, k, tile):
    """Shapes whose tile count selects each tile size (at least 384 tiles of
    128 x 128, else at least 256 of 64 x 128, else 64 x 64), ragged where
    possible; outputs checked on sampled blocks, the tile edges among them."""
    rng = np.random.default_rng(4600 + n)
    w16 = oracle_mod.f16_cvt((rng.standard_normal((n, k)) * 0.05).astype(np.float32))
    x16 = oracle_mod.f16_cvt(rng.standard_normal((m, k)).astype(np.float32))
    _say("f16 gemm m=%d n=%d k=%d (%s tiles)" % (m, n, k, tile))
    y = _gemm_gpu(w16, x16, m, n, k)
    rows = np.r_[0:70, n // 2 - 70:n // 2 + 70, n - 70:n]
    vecs = np.r_[0:70, m - 70:m]
    y_ref, bound = oracle_mod.f16_gemm(w16[rows], x16[vecs])
    _check_gemm(y[np.ix_(vecs, rows)], y_ref, bound, k, "%s sample" % tile)


def test_f16_gemm_integer_operands_exact(oracle_mod):
    """Small integers: every partial sum is an integer below 2^24, so the
    f32 accumulation is exact and y must equal the integer product."""
    rng = np.random.default_rng(4401)
    m, n, k = 96, 200, 512
    wi = rng.integers(-8, 9, size=(n, k))
    xi = rng.integers(-8, 9, size=(m, k))
    y = _gemm_gpu(oracle_mod.f16_cvt(wi.astype(np.float32)),
                  oracle_mod.f16_cvt(xi.astype(np.float32)), m, n, k)
    assert np.array_equal(y.astype(np.int64), xi @ wi.T)


def test_prefill_from_q4k_weights(oracle_mod):
    """The whole prefill path on Q4_K weights: the mirror, then the f32
    activations converted into a scratch and multiplied (q4k_f16_gemm_f32x),
    at the prefill batch of the pages (m = 512) on 4096 x 4096 weights;
    outputs checked on sampled blocks of rows and vectors."""
    n, k, m = 4096, 4096, 512
    w, _ = synth.make_inputs(n, k, 1, seed=4501)
    x = np.random.default_rng(4502).standard_normal((m, k)).astype(np.float32)
    _say("prefill m=%d n=%d k=%d" % (m, n, k))
    w_d = torch.from_numpy(w).cuda()
    w16_d = torch.empty((n, k), dtype=torch.int16, device="cuda")
    q4k.q4k_mirror_f16(w_d, w16_d, n, k)
    x_d = torch.from_numpy(x).cuda()
    xh_d = torch.empty((m, k), dtype=torch.int16, device="cuda")
    y_d = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    q4k.q4k_f16_gemm_f32x(w16_d, x_d, xh_d, y_d, m, n, k)
    torch.cuda.synchronize()
    y = y_d.cpu().numpy()
    rows = np.r_[0:40, 2000:2040, n - 40:n]
    vecs = np.r_[0:16, 250:266, m - 16:m]
    w16 = oracle_mod.mirror_f16(w, 4, n, k)
    x16 = oracle_mod.f16_cvt(x)
    assert np.array_equal(xh_d.cpu().numpy().view(np.uint16), x16)
    y_ref, bound = oracle_mod.f16_gemm(w16[rows], x16[vecs])
    _check_gemm(y[np.ix_(vecs, rows)], y_ref, bound, k, "prefill sample")

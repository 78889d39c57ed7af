"""GPU parity of the integer-dot variant with Q8 activations (q4k_gemv_q8,
q4k_quantize_q8; realizar 0.8.5, modules_utilities.rs,
`preload_hw_dp4a_modules`).

The quantization is integer work decided in f32 on both sides: its codes
and scales must equal the oracle's bit for bit (oracle.quantize_q8).  The
GEMV is checked twice: against the oracle's exact GEMV of the quantized x
(within 2^-23 |y| + 1e-9 sum|w||d q|: only f64 scaling and the final f32
rounding differ), and against the exact GEMV of the f32 x within the
variant's own stated tolerance, sum_e |w_e| (d_b/2 (1 + 2^-19) + 2^-20 |x_e|)
+ 2^-23 |y_ref|.
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


def _quantize_gpu(x):
    m, k = x.shape
    x_d = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    q_d = torch.full((m, k), 99, dtype=torch.int8, device="cuda")
    d_d = torch.full((m, k // 32), 12345.0, dtype=torch.float32, device="cuda")
    q4k.q4k_quantize_q8(x_d, q_d, d_d, k, m)
    torch.cuda.synchronize()
    return q_d.cpu().numpy(), d_d.cpu().numpy()


def _x_cases(rng):
    k = 2048
    spread = (rng.standard_normal((2, k)) *
              np.exp2(rng.integers(-40, 41, size=(2, k // 32, 1))).repeat(32, axis=2).reshape(2, k))
    mixed = rng.standard_normal((2, k)) * np.exp2(rng.integers(-20, 21, size=(2, k)))
    z = rng.standard_normal((2, k))
    z[:, 64:96] = 0.0
    z[0, 130] = 1e30
    z[1, 200:232] = 1e-40              # subnormal block
    return [spread, mixed, z, rng.standard_normal((3, 4096)) * 3.0]


def test_quantize_matches_oracle(oracle_mod):
    rng = np.random.default_rng(1201)
    for x in _x_cases(rng):
        x = x.astype(np.float32)
        _say("q8 quantize m=%d k=%d" % x.shape)
        q, d = _quantize_gpu(x)
        q_ref, d_ref = oracle_mod.quantize_q8(x)
        assert np.array_equal(q, q_ref)
        assert np.array_equal(d.view(np.uint32), d_ref.view(np.uint32))


def test_quantize_non_finite_blocks(oracle_mod):
    x = np.ones((1, 128), np.float32)
    x[0, 3] = np.nan
    x[0, 40] = np.inf
    x[0, 70] = -np.inf
    q, d = _quantize_gpu(x)
    q_ref, d_ref = oracle_mod.quantize_q8(x)
    assert np.array_equal(q, q_ref)
    assert np.isnan(d[0, 0]) and np.isinf(d[0, 1]) and np.isinf(d[0, 2])
    assert np.array_equal(d[0, 3:], d_ref[0, 3:])


def _run_q8(w_d, x, n, k):
    x_d = torch.from_numpy(np.ascontiguousarray(x.reshape(1, k))).cuda()
    y_d = torch.full((1, n), 7.0, dtype=torch.float32, device="cuda")
    q4k.q4k_gemv_q8(w_d, x_d, y_d, n, k, 1)
    torch.cuda.synchronize()
    return y_d.cpu().numpy()[0].astype(np.float64)


def _check_q8(oracle_mod, w, x, n, k, what):
    w_d = torch.from_numpy(w).cuda()
    y = _run_q8(w_d, x, n, k)
    q, d = oracle_mod.quantize_q8(x.reshape(1, k))
    yq, bq = oracle_mod.gemv_q8(w, q, d, n)
    yq, bq = yq[0], bq[0]
    assert np.all(np.abs(y - yq) <= 2.0 ** -23 * np.abs(yq) + 1e-9 * bq), what
    # the variant's own tolerance against the exact GEMV of the f32 x
    y_ref, _ = oracle_mod.gemv(w, x.reshape(1, k), n)
    y_ref = y_ref[0]
    aw = np.abs(oracle_mod.dequant(w, n, k).astype(np.float64))
    xa = np.abs(x.reshape(k).astype(np.float64))
    dq = np.repeat(d[0].astype(np.float64), 32)
    tol = aw @ (dq / 2 * (1 + 2.0 ** -19) + 2.0 ** -20 * xa) + 2.0 ** -23 * np.abs(y_ref)
    err = np.abs(y - y_ref)
    assert np.all(err <= tol), (what, float((err / tol).max()))
    return float((err / np.maximum(tol, 1e-300)).max())


@pytest.mark.parametrize("index", [0, 1, 2, 3])
def test_q8_gemv_workloads(oracle_mod, index):
    wl, w, x = synth.workload_inputs(index)
    _say("q8 gemv workload %d (%s)" % (index, wl.name))
    r = _check_q8(oracle_mod, w, x[0], wl.n, wl.k, wl.name)
    _say("  worst error / stated tolerance %.3g" % r)


@pytest.mark.parametrize("n,k", [(1, 256), (17, 1280), (300, 4096), (257, 11008), (33, 2304),
                                 (64, 16384)])
def test_q8_gemv_shapes(oracle_mod, n, k):
    w, x = synth.make_inputs(n, k, 1, seed=n * 53 + k)
    _say("q8 gemv n=%d k=%d" % (n, k))
    _check_q8(oracle_mod, w, x[0], n, k, "n=%d k=%d" % (n, k))


def test_q8_gemv_x_magnitudes(oracle_mod):
    n, k = 48, 4096
    rng = np.random.default_rng(1202)
    w, _ = synth.make_inputs(n, k, 1, seed=1203)
    x = (rng.standard_normal(k) * np.exp2(rng.integers(-60, 61, size=k // 32)).repeat(32)).astype(
        np.float32)
    _say("q8 gemv, block magnitudes 2^-60 .. 2^60")
    _check_q8(oracle_mod, w, x, n, k, "block magnitudes")


def test_q8_gemv_non_finite_x_gives_nan(oracle_mod):
    n, k = 40, 2048
    w, x = synth.make_inputs(n, k, 1, seed=1204)
    x = x[0].copy()
    x[77] = np.inf
    y = _run_q8(torch.from_numpy(w).cuda(), x, n, k)
    assert np.all(np.isnan(y))
    x[77] = np.nan
    y = _run_q8(torch.from_numpy(w).cuda(), x, n, k)
    assert np.all(np.isnan(y))


def test_q8_refusals_on_device():
    n, k = 64, 2048
    w, x = synth.make_inputs(n, k, 2, seed=1205)
    w_d = torch.from_numpy(w).cuda()
    x_d = torch.from_numpy(x).cuda()
    y_d = torch.full((2, n), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_gemv_q8(w_d, x_d, y_d, n, k, 2)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((y_d == 7.0).all())

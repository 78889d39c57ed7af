"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars:
  * q4k_dequantize: bit-exact against the oracle's f32 weights.
  * q4k_gemv: |y - y_ref| <= 1e-5 * sum_c |w||x| per output, y_ref the
    oracle's f64 dot of the dequantized weights (a zero bound demands y == 0).
  * single-stage and K-chunked variants, every row/wave/x-placement option,
    and m-batched vs m separate m = 1 calls: bit-identical y (the pages hold
    batched kernels bit-exact against their GEMVs: turbospark-runtime 0.1.0,
    real_forward_dispatch.rs, doc of `encode_gemm_any`).
All five workloads run at full size; the oracle computes every output.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import checks  # noqa: E402

from block_quantized_decode_q4_amd import q4k, synth  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    q4k.load_library()
    yield


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gemv(w_d, x_np, n, k, m, **opts):
    x_d = dev(x_np.reshape(m, k))
    y_d = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    if opts:
        q4k.q4k_gemv_ex(w_d, x_d, y_d, n, k, m, **opts)
    else:
        q4k.q4k_gemv(w_d, x_d, y_d, n, k, m)
    torch.cuda.synchronize()
    return y_d.cpu().numpy()


def assert_within(y, y_ref, bound, what):
    """The rule of tests/checks.py: within 1e-5 * sum|w||x| of every finite
    exact result (a NaN or infinity in y fails), non-finite where it is."""
    return checks.assert_y(y, y_ref, bound, what)


_cache = {}


def workload(i, oracle_mod):
    if i not in _cache:
        wl, w, x = synth.workload_inputs(i)
        y_ref, bound = oracle_mod.gemv(w, x, wl.n)
        _cache.clear()
        _cache[i] = (wl, w, x, y_ref, bound)
    return _cache[i]


@pytest.mark.parametrize("i", range(5))
def test_dequant_bit_exact_workload(oracle_mod, i):
    wl, w, x, _, _ = workload(i, oracle_mod)
    _say("dequant workload %d n=%d k=%d" % (i, wl.n, wl.k))
    w_d = dev(w)
    out = torch.empty((wl.n, wl.k), dtype=torch.float32, device="cuda")
    q4k.q4k_dequantize(w_d, out, wl.n, wl.k)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle_mod.dequant(w, wl.n, wl.k)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("i", range(5))
def test_gemv_workload(oracle_mod, i):
    wl, w, x, y_ref, bound = workload(i, oracle_mod)
    _say("gemv workload %d n=%d k=%d m=%d" % (i, wl.n, wl.k, wl.m))
    w_d = dev(w)
    y = run_gemv(w_d, x, wl.n, wl.k, wl.m)
    worst = assert_within(y, y_ref, bound, "workload %d" % i)
    _say("  worst |err|/bound = %.3e" % worst)


def test_load_then_gemv(oracle_mod):
    wl, w, x, y_ref, bound = workload(1, oracle_mod)
    w_d = torch.empty(w.size, dtype=torch.uint8, device="cuda")
    q4k.q4k_load(w_d, w, wl.n, wl.k)
    assert torch.equal(w_d.cpu(), torch.from_numpy(w))
    y = run_gemv(w_d, x, wl.n, wl.k, wl.m)
    assert_within(y, y_ref, bound, "after q4k_load")


VARIANTS = [
    dict(kernel=1, variant=1),
    dict(kernel=1, variant=2, spans_per_chunk=1),
    dict(kernel=1, variant=2, spans_per_chunk=2),
    dict(kernel=1, variant=1, rows_per_wave=1),
    dict(kernel=1, variant=1, rows_per_wave=4),
    dict(kernel=1, variant=1, waves_per_block=8),
    dict(kernel=1, variant=2, spans_per_chunk=1, rows_per_wave=4, waves_per_block=8),
    dict(kernel=1, variant=1, rows_per_block=5, rows_per_wave=2),
    dict(kernel=1, variant=2, spans_per_chunk=1, rows_per_block=3, rows_per_wave=4),
    dict(kernel=1, variant=1, rows_per_block=1000, rows_per_wave=4),
    dict(kernel=1, variant=1, x_in_registers=2),
]


STREAM_VARIANTS = [
    dict(kernel=2),
    dict(kernel=2, ring_depth=2, rows_per_task=7),
    dict(kernel=2, ring_depth=2, rows_per_task=64, waves_per_block=4),
    dict(kernel=2, ring_depth=4, rows_per_task=16, waves_per_block=8),
    dict(kernel=2, ring_depth=3, rows_per_task=1, waves_per_block=4, rows_per_block=3),
    dict(kernel=2, ring_depth=1, rows_per_task=3, waves_per_block=8),
    dict(kernel=2, variant=2, spans_per_chunk=1, rows_per_task=5, rows_per_block=37),
    dict(kernel=2, variant=1, rows_per_task=33, rows_per_block=200),
]


@pytest.mark.parametrize("i", [0, 1, 2, 3])
def test_streaming_kernel_variants(oracle_mod, i):
    """The streaming kernel: within tolerance and bit-identical across its
    launch options (each row-span partial is one wave's fixed sequence; spans
    are added in a fixed order)."""
    wl, w, x, y_ref, bound = workload(i, oracle_mod)
    w_d = dev(w)
    base = None
    for opts in STREAM_VARIANTS:
        _say("workload %d streaming %r" % (i, opts))
        y = run_gemv(w_d, x, wl.n, wl.k, wl.m, **opts)
        assert_within(y, y_ref, bound, "streaming %r" % opts)
        if base is None:
            base = y
        else:
            assert np.array_equal(y.view(np.uint32), base.view(np.uint32)), opts


@pytest.mark.parametrize("n,k", [(1, 256), (5, 768), (130, 4096 + 2304), (65, 12544), (3, 65536)])
def test_streaming_kernel_shapes(oracle_mod, n, k):
    w, x = synth.make_inputs(n, k, 1, seed=n + 3 * k)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    for opts in STREAM_VARIANTS[:3]:
        _say("streaming n=%d k=%d %r" % (n, k, opts))
        y = run_gemv(w_d, x, n, k, 1, **opts)
        assert_within(y, y_ref, bound, "streaming n=%d k=%d %r" % (n, k, opts))


# line-streamed int8 matrix-core kernel (k a multiple of 2048): its sums run
# in the same order for every launch geometry with the same column grouping,
# so those launches are bit-identical
LINES_VARIANTS = [
    dict(kernel=4),
    dict(kernel=4, cols_per_task=8),
    dict(kernel=4, waves_per_block=4, rows_per_block=48),
    dict(kernel=4, waves_per_block=16, rows_per_block=320, cols_per_task=8),
    dict(kernel=4, rows_per_block=40),
    dict(kernel=4, waves_per_block=4, rows_per_block=16),
    dict(kernel=4, ring_depth=9),
    dict(kernel=4, ring_depth=9, cols_per_task=8, rows_per_block=16),
    dict(kernel=4, ring_depth=9, waves_per_block=4, rows_per_block=80),
]


def _lines_auto_cols(n, k, m, opts):
    """The line-streamed kernel's automatic column grouping: whole rows when
    the workgroup has a 16-row tile for every wave or when the per-slab row
    sums do not fit the LDS, else one slab of 8 columns."""
    S = k // 256
    ntiles = (n + 15) // 16
    rpb = opts.get("rows_per_block") or 16 * ((ntiles + 255) // 256)
    nw = opts.get("waves_per_block", 8)
    fits = (S * m + 1) * 1264 + nw * 4352 + (S // 8) * rpb * 8 * m <= 160 * 1024
    return S if (rpb // 16 >= nw or not fits) else 8


def _lines_check(w_d, w, x, n, k, y_ref, bound, what):
    S = k // 256
    firsts = {}
    for opts in LINES_VARIANTS:
        _say("%s line-streamed %r" % (what, opts))
        try:
            y = run_gemv(w_d, x, n, k, 1, **opts)
        except q4k.Q4KError as e:
            # refused: a task's column group must divide the slabs of a row,
            # the whole staged x (1264 bytes per superblock column) plus the
            # line rings (4352 bytes per wave) and row sums must fit the
            # 160 KiB LDS; 16-wave workgroups are refused
            nw = opts.get("waves_per_block", 8)
            bad_group = "cols_per_task" in opts and (S // 8) % (opts["cols_per_task"] // 8) != 0
            ncg = (S // 8) // (opts["cols_per_task"] // 8) if "cols_per_task" in opts else 1
            rpb = opts.get("rows_per_block", 16 * (((n + 15) // 16 + 255) // 256))
            ysum = ncg * rpb * 8 if ncg > 1 else 0
            too_big = (S + 1) * 1264 + nw * 4352 + ysum > 160 * 1024 or nw == 16
            assert e.rc == q4k.Q4K_ERR_UNSUPPORTED and (bad_group or too_big), opts
            continue
        assert_within(y, y_ref, bound, "%s line-streamed %r" % (what, opts))
        cpt = opts.get("cols_per_task") or _lines_auto_cols(n, k, 1, opts)
        if cpt in firsts:
            assert np.array_equal(y.view(np.uint32), firsts[cpt].view(np.uint32)), opts
        else:
            firsts[cpt] = y


@pytest.mark.parametrize("i", [1, 2, 3])
def test_lines_kernel_workloads(oracle_mod, i):
    wl, w, x, y_ref, bound = workload(i, oracle_mod)
    _lines_check(dev(w), w, x, wl.n, wl.k, y_ref, bound, "workload %d" % i)


@pytest.mark.parametrize("n,k", [(1, 2048), (17, 4096), (130, 14336), (3, 65536), (257, 2048),
                                 (33, 18432)])
def test_lines_kernel_shapes(oracle_mod, n, k):
    w, x = synth.make_inputs(n, k, 1, seed=n + 11 * k)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    _lines_check(dev(w), w, x, n, k, y_ref, bound, "n=%d k=%d" % (n, k))


@pytest.mark.parametrize("n,k,m", [(300, 4096, 2), (33, 2048, 2), (40, 8192, 2), (130, 6144, 2)])
def test_lines_kernel_batched(oracle_mod, n, k, m):
    """Two vectors in one launch: within tolerance, and bit-identical to two
    single-vector launches of the same kernel (each vector's sums run in
    the same order)."""
    w, x = synth.make_inputs(n, k, m, seed=n * 31 + k + m)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    _say("line-streamed batched n=%d k=%d m=%d" % (n, k, m))
    y = run_gemv(w_d, x, n, k, m, kernel=4)
    assert_within(y, y_ref, bound, "line-streamed m=%d" % m)
    for b in range(m):
        y1 = run_gemv(w_d, x[b:b + 1], n, k, 1, kernel=4)
        assert np.array_equal(y1[0].view(np.uint32), y[b].view(np.uint32)), b


def test_lines_kernel_batched_workload(oracle_mod):
    """The batched workload's vectors two at a time on the per-vector
    matrix-core kernel (one MFMA group per vector takes at most two)."""
    wl, w, x, y_ref, bound = workload(4, oracle_mod)
    w_d = dev(w)
    _say("line-streamed batched workload 4, two vectors per launch")
    with pytest.raises(q4k.Q4KError) as e:
        run_gemv(w_d, x, wl.n, wl.k, wl.m, kernel=4)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    for b in range(0, wl.m, 2):
        y2 = run_gemv(w_d, x[b:b + 2], wl.n, wl.k, 2, kernel=4)
        assert_within(y2, y_ref[b:b + 2], bound[b:b + 2], "line-streamed workload 4 pair %d" % b)


@pytest.mark.parametrize("n,k,m", [(300, 4096, 1), (300, 4096, 2), (17, 2048, 3), (130, 2048, 8),
                                   (64, 2048, 5), (33, 2048, 8), (40, 4096, 4), (1, 2048, 6)])
def test_sub_kernel(oracle_mod, n, k, m):
    """The sub-block kernel: within tolerance, bit-identical to m
    single-vector launches of itself, and across workgroup shapes with the
    same column grouping."""
    w, x = synth.make_inputs(n, k, m, seed=n * 17 + k + 3 * m)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    _say("sub-block kernel n=%d k=%d m=%d" % (n, k, m))
    y = run_gemv(w_d, x, n, k, m, kernel=5, cols_per_task=8)
    assert_within(y, y_ref, bound, "sub-block m=%d" % m)
    for b in range(m):
        y1 = run_gemv(w_d, x[b:b + 1], n, k, 1, kernel=5, cols_per_task=8)
        assert np.array_equal(y1[0].view(np.uint32), y[b].view(np.uint32)), b
    for opts in (dict(rows_per_block=48), dict(rows_per_block=16), dict(rows_per_block=200)):
        y2 = run_gemv(w_d, x, n, k, m, kernel=5, cols_per_task=8, **opts)
        assert np.array_equal(y2.view(np.uint32), y.view(np.uint32)), opts
    y3 = run_gemv(w_d, x, n, k, m, kernel=5, cols_per_task=k // 256)
    assert_within(y3, y_ref, bound, "sub-block whole rows m=%d" % m)


def test_sub_kernel_workload(oracle_mod):
    """The batched workload (14336 x 4096, eight vectors): its whole x stage
    (33 groups of 4752 bytes) and the rings exceed the LDS, so kernel 5 is
    refused; the automatic plan (the column window, kernel 7) and kernel 6
    agree bit for bit."""
    wl, w, x, y_ref, bound = workload(4, oracle_mod)
    _say("sub-block kernels workload 4")
    with pytest.raises(q4k.Q4KError) as ei:
        run_gemv(dev(w), x, wl.n, wl.k, wl.m, kernel=5)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    y = run_gemv(dev(w), x, wl.n, wl.k, wl.m)
    assert_within(y, y_ref, bound, "automatic workload 4")
    y6 = run_gemv(dev(w), x, wl.n, wl.k, wl.m, kernel=6)
    assert np.array_equal(y6.view(np.uint32), y.view(np.uint32))


# kernel 6: the sub-block decode with x converted one superblock column at a
# time by each wave for itself (no whole x stage), automatic for batches
# whose whole x stage does not fit the LDS.  Its digits, MFMAs and sums are
# those of kernel 5 in the same order, so where both run with the same
# column grouping they give bit-identical y.
@pytest.mark.parametrize("n,k,m", [(300, 4096, 2), (17, 2048, 3), (130, 4096, 8), (64, 4096, 5),
                                   (33, 2048, 8), (40, 8192, 4), (1, 2048, 6), (64, 4096, 1),
                                   # no whole x stage fits: automatic kernel 6
                                   (130, 14336, 8), (48, 28672, 3), (257, 16384, 4),
                                   (20, 22528, 7)])
def test_jit_kernel(oracle_mod, n, k, m):
    w, x = synth.make_inputs(n, k, m, seed=n * 29 + k + 5 * m)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    _say("per-wave x kernel n=%d k=%d m=%d" % (n, k, m))
    y = run_gemv(w_d, x, n, k, m, kernel=6, cols_per_task=8)
    assert_within(y, y_ref, bound, "per-wave x m=%d" % m)
    for b in range(m):                          # batched == m single-vector launches
        y1 = run_gemv(w_d, x[b:b + 1], n, k, 1, kernel=6, cols_per_task=8)
        assert np.array_equal(y1[0].view(np.uint32), y[b].view(np.uint32)), b
    try:
        y5 = run_gemv(w_d, x, n, k, m, kernel=5, cols_per_task=8)
    except q4k.Q4KError as e:
        assert e.rc == q4k.Q4K_ERR_UNSUPPORTED
    else:
        assert np.array_equal(y5.view(np.uint32), y.view(np.uint32))
    for opts in (dict(rows_per_block=48, cols_per_task=8), dict(rows_per_block=16, cols_per_task=8),
                 dict(rows_per_block=100, cols_per_task=8)):
        y2 = run_gemv(w_d, x, n, k, m, kernel=6, **opts)
        assert np.array_equal(y2.view(np.uint32), y.view(np.uint32)), opts
    y3 = run_gemv(w_d, x, n, k, m, kernel=6, cols_per_task=k // 256)
    assert_within(y3, y_ref, bound, "per-wave x whole rows m=%d" % m)
    if m > 1:
        y4 = run_gemv(w_d, x, n, k, m)         # automatic kernel
        assert_within(y4, y_ref, bound, "automatic m=%d k=%d" % (m, k))


@pytest.mark.parametrize("n,k,m", [(17, 1280, 3), (130, 11008, 8), (33, 4352, 2), (257, 5120, 5),
                                   (48, 13824, 4), (5, 768, 6), (16, 2304, 7), (1, 256, 2),
                                   (300, 3328, 8)])
def test_sub_kernels_partial_slabs(oracle_mod, n, k, m):
    """Kernels 5 and 6 on rows of partial slabs (k not a multiple of 2048:
    four-line rings, per-row start offsets): within tolerance, bit-identical
    to each other with the same column grouping, and the automatic plan."""
    w, x = synth.make_inputs(n, k, m, seed=n * 31 + k + 7 * m)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    _say("partial-slab sub-block kernels n=%d k=%d m=%d" % (n, k, m))
    y6 = run_gemv(w_d, x, n, k, m, kernel=6, cols_per_task=8)
    assert_within(y6, y_ref, bound, "per-wave x partial slabs m=%d" % m)
    for b in range(m):                          # batched == m single-vector launches
        y1 = run_gemv(w_d, x[b:b + 1], n, k, 1, kernel=6, cols_per_task=8)
        assert np.array_equal(y1[0].view(np.uint32), y6[b].view(np.uint32)), b
    try:
        y5 = run_gemv(w_d, x, n, k, m, kernel=5, cols_per_task=8)
    except q4k.Q4KError as e:
        assert e.rc == q4k.Q4K_ERR_UNSUPPORTED
    else:
        assert np.array_equal(y5.view(np.uint32), y6.view(np.uint32))
    nslabs = (k // 256 + 7) // 8
    for opts in (dict(rows_per_block=48), dict(cols_per_task=8 * nslabs)):
        y2 = run_gemv(w_d, x, n, k, m, kernel=6, **opts)
        assert_within(y2, y_ref, bound, "per-wave x partial slabs %r" % opts)
    y4 = run_gemv(w_d, x, n, k, m)             # automatic kernel
    assert_within(y4, y_ref, bound, "automatic partial slabs m=%d k=%d" % (m, k))


# kernel 7: the sub-block decode with x converted once per workgroup, one
# column ahead, into a two-column window of every slab (waves in step, one
# LDS barrier per column).  Per column and vector its digits, MFMAs and sums
# are those of kernels 5 and 6, so with one slab per task the three agree
# bit for bit.  Small n leaves waves without a task: they still convert and
# meet the barriers.
@pytest.mark.parametrize("n,k,m", [(300, 4096, 8), (130, 4096, 4), (64, 8192, 2), (17, 2048, 3),
                                   (1, 4096, 16), (257, 16384, 1), (40, 4096, 12), (3, 6144, 5),
                                   (1000, 8192, 6)])
def test_window_kernel(oracle_mod, n, k, m):
    w, x = synth.make_inputs(n, k, m, seed=n * 43 + k + 3 * m)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    _say("window kernel n=%d k=%d m=%d" % (n, k, m))
    y = run_gemv(w_d, x, n, k, m, kernel=7)
    assert_within(y, y_ref, bound, "window m=%d" % m)
    for b in range(m):                          # batched == m single-vector launches
        y1 = run_gemv(w_d, x[b:b + 1], n, k, 1, kernel=7)
        assert np.array_equal(y1[0].view(np.uint32), y[b].view(np.uint32)), b
    y6 = run_gemv(w_d, x, n, k, m, kernel=6, cols_per_task=8)
    assert np.array_equal(y6.view(np.uint32), y.view(np.uint32))
    try:
        y5 = run_gemv(w_d, x, n, k, m, kernel=5, cols_per_task=8)
    except q4k.Q4KError as e:
        assert e.rc == q4k.Q4K_ERR_UNSUPPORTED
    else:
        assert np.array_equal(y5.view(np.uint32), y.view(np.uint32))
    ncg = k // 2048
    for rpb in (16, 32, 48):
        if (rpb + 15) // 16 * ncg > 8:
            continue
        y2 = run_gemv(w_d, x, n, k, m, kernel=7, rows_per_block=rpb)
        assert np.array_equal(y2.view(np.uint32), y.view(np.uint32)), rpb


def test_window_kernel_workload(oracle_mod):
    """The batched workload (14336 x 4096, eight vectors) on its automatic
    plan, the column window."""
    wl, w, x, y_ref, bound = workload(4, oracle_mod)
    assert q4k.q4k_plan(wl.n, wl.k, wl.m).kernel == 7
    _say("window kernel workload 4")
    y = run_gemv(dev(w), x, wl.n, wl.k, wl.m)
    assert_within(y, y_ref, bound, "window workload 4")


def test_jit_kernel_ffn_down_batch8(oracle_mod):
    """The FFN-down shape (4096 x 14336) with eight vectors: the automatic
    plan (kernel 6, no whole x stage fits) against the oracle."""
    n, k, m = 4096, 14336, 8
    w, x = synth.make_inputs(n, k, m, seed=4096 + 14336 + 8)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    _say("automatic n=%d k=%d m=%d" % (n, k, m))
    y = run_gemv(dev(w), x, n, k, m)
    assert_within(y, y_ref, bound, "automatic FFN-down m=8")


def test_jit_kernel_x_dynamic_range(oracle_mod):
    n, k = 40, 4096
    rng = np.random.default_rng(77)
    w, _ = synth.make_inputs(n, k, 1, seed=321)
    xs = _x_cases(rng, k)
    y_ref, bound = oracle_mod.gemv(w, xs, n)
    y = run_gemv(dev(w), xs, n, k, 2, kernel=6)
    assert_within(y, y_ref, bound, "per-wave x dynamic-range x")


# line-streamed vector-ALU kernel (m = 1, any k): integer dot products with x
# broadcast across the tile's rows by DPP; rows of a whole number of slabs
# (k a multiple of 2048) take the two-line rings, other rows four-line rings
# and per-row start offsets.  Its sums run in the same order for every launch
# geometry with the same column grouping, so those launches are bit-identical.
DOT4_VARIANTS = [
    dict(kernel=3),
    dict(kernel=3, cols_per_task=8),
    dict(kernel=3, waves_per_block=4, rows_per_block=48),
    dict(kernel=3, waves_per_block=16, rows_per_block=320, cols_per_task=8),
    dict(kernel=3, rows_per_block=40),
    dict(kernel=3, waves_per_block=4, rows_per_block=16),
    dict(kernel=3, ring_depth=9),
    dict(kernel=3, ring_depth=9, cols_per_task=8, rows_per_block=16),
    dict(kernel=3, ring_depth=9, waves_per_block=4, rows_per_block=80),
]


def _dot4_auto_cols(n, k, opts):
    """Automatic column grouping of the vector-ALU line-streamed kernel:
    whole rows when the workgroup has a tile for every wave or when the
    per-slab row sums do not fit the LDS, else one slab of 8 columns."""
    S = k // 256
    nslabs = (S + 7) // 8
    ntiles = (n + 15) // 16
    rpb = opts.get("rows_per_block") or 16 * ((ntiles + 255) // 256)
    nw = opts.get("waves_per_block", 8)
    fits = S * 1200 + nw * _dot4_ring(S) + nslabs * rpb * 8 <= 160 * 1024
    return 8 * nslabs if (rpb // 16 >= nw or not fits) else 8


def _dot4_ring(S):
    """LDS bytes of one wave's line rings: two lines per row for rows of
    whole slabs, four otherwise (16 rows, 16 bytes of padding per row)."""
    return 16 * (2 * 128 + 16) if S % 8 == 0 else 16 * (4 * 128 + 16)


def _dot4_check(w_d, x, n, k, y_ref, bound, what):
    S = k // 256
    nslabs = (S + 7) // 8
    firsts = {}
    for opts in DOT4_VARIANTS:
        _say("%s vector-ALU line-streamed %r" % (what, opts))
        nw = opts.get("waves_per_block", 8)
        try:
            y = run_gemv(w_d, x, n, k, 1, **opts)
        except q4k.Q4KError as e:
            # refused: a task's column group must divide the slabs of a row,
            # the staged x (1200 bytes per superblock column) plus the line
            # rings and row sums must fit the 160 KiB LDS, x takes at most four
            # groups per lane, 16-wave workgroups are refused
            # 16-element groups per lane, rows of partial slabs keep three
            # lines in flight
            bad_group = "cols_per_task" in opts and nslabs % (opts["cols_per_task"] // 8) != 0
            # staged x: 1200 bytes per column; f64 row sums per slab group
            ncg = nslabs // (opts["cols_per_task"] // 8) if "cols_per_task" in opts else 1
            rpb = opts.get("rows_per_block", 16 * (((n + 15) // 16 + 255) // 256))
            ysum = ncg * rpb * 8 if ncg > 1 else 0
            too_big = (S * 1200 + nw * _dot4_ring(S) + ysum > 160 * 1024
                       or S * 16 > 4 * 64 * nw or nw == 16)
            bad_ring = S % 8 != 0 and opts.get("ring_depth", 3) != 3
            assert e.rc == q4k.Q4K_ERR_UNSUPPORTED and (bad_group or too_big or bad_ring), opts
            continue
        assert_within(y, y_ref, bound, "%s vector-ALU line-streamed %r" % (what, opts))
        cpt = opts.get("cols_per_task") or _dot4_auto_cols(n, k, opts)
        if cpt in firsts:
            assert np.array_equal(y.view(np.uint32), firsts[cpt].view(np.uint32)), opts
        else:
            firsts[cpt] = y


@pytest.mark.parametrize("i", [0, 1, 2, 3])
def test_dot4_kernel_workloads(oracle_mod, i):
    wl, w, x, y_ref, bound = workload(i, oracle_mod)
    _dot4_check(dev(w), x, wl.n, wl.k, y_ref, bound, "workload %d" % i)


@pytest.mark.parametrize("n,k", [(1, 2048), (17, 4096), (130, 14336), (3, 65536), (257, 2048),
                                 (33, 18432), (20, 24576),
                                 # rows of partial slabs: any start offset in a line
                                 (1, 256), (5, 768), (17, 1280), (33, 4352), (130, 11008),
                                 (257, 5120), (16, 2304), (48, 13824), (300, 3328),
                                 # a 16-row tile for each of the 8 waves of a
                                 # workgroup: whole rows per task
                                 (28688, 1280), (28720, 2560)])
def test_dot4_kernel_shapes(oracle_mod, n, k):
    w, x = synth.make_inputs(n, k, 1, seed=n + 13 * k)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    _dot4_check(dev(w), x, n, k, y_ref, bound, "n=%d k=%d" % (n, k))


@pytest.mark.parametrize("n,k", [(64, 2048), (33, 4096), (40, 1280)])
def test_dot4_kernel_x_dynamic_range(oracle_mod, n, k):
    rng = np.random.default_rng(n * k + 1)
    w, _ = synth.make_inputs(n, k, 1, seed=n + k + 1)
    xs = _x_cases(rng, k)
    w_d = dev(w)
    for b in range(xs.shape[0]):
        x = xs[b:b + 1]
        y_ref, bound = oracle_mod.gemv(w, x, n)
        for opts in DOT4_VARIANTS[:2]:
            _say("vector-ALU dynamic range n=%d k=%d case %d %r" % (n, k, b, opts))
            y = run_gemv(w_d, x, n, k, 1, **opts)
            assert_within(y, y_ref, bound, "vector-ALU x case %d %r" % (b, opts))


def test_dot4_kernel_refusals():
    """Shapes the vector-ALU line-streamed kernel cannot take are refused
    without launching: several vectors, rows not 128-byte aligned, x larger
    than four groups of 16 per lane."""
    n = 8
    w, x = synth.make_inputs(n, 2048, 2, seed=8)
    y_d = torch.zeros((2, n), dtype=torch.float32, device="cuda")
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q4k_gemv_ex(dev(w), dev(x), y_d, n, 2048, 2, kernel=3)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    w_d = torch.zeros(w.size + 128, dtype=torch.uint8, device="cuda")
    w_d[16:16 + w.size] = torch.from_numpy(w).cuda()
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q4k_gemv_ex(w_d.data_ptr() + 16, dev(x[:1]), y_d, n, 2048, 1, kernel=3)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    w2, x2 = synth.make_inputs(n, 65536, 1, seed=9)
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q4k_gemv_ex(dev(w2), dev(x2), y_d, n, 65536, 1, kernel=3, waves_per_block=8)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(y_d).item() == 0


def test_sub_kernel_x_dynamic_range(oracle_mod):
    n, k = 40, 4096
    rng = np.random.default_rng(99)
    w, _ = synth.make_inputs(n, k, 1, seed=123)
    xs = _x_cases(rng, k)
    y_ref, bound = oracle_mod.gemv(w, xs, n)
    y = run_gemv(dev(w), xs, n, k, 2, kernel=5)
    assert_within(y, y_ref, bound, "sub-block dynamic-range x")


def test_lines_kernel_refusals():
    """Shapes and pointers the line-streamed kernel cannot take are refused
    without launching (k not a multiple of 2048, rows not 128-byte aligned)."""
    n, k = 8, 2048
    w, x = synth.make_inputs(n, k, 1, seed=5)
    w_d = torch.zeros(w.size + 128, dtype=torch.uint8, device="cuda")
    w_d[16:16 + w.size] = torch.from_numpy(w).cuda()
    x_d = dev(x)
    y_d = torch.zeros((1, n), dtype=torch.float32, device="cuda")
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q4k_gemv_ex(w_d.data_ptr() + 16, x_d, y_d, n, k, 1, kernel=4)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    w2, x2 = synth.make_inputs(n, 1024, 1, seed=6)
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q4k_gemv_ex(dev(w2), dev(x2), y_d, n, 1024, 1, kernel=4)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    # at most two vectors, and the staged x of every vector must fit the
    # LDS: 72 columns x 2 vectors do not
    w3, x3 = synth.make_inputs(n, 8192, 5, seed=7)
    y3 = torch.zeros((5, n), dtype=torch.float32, device="cuda")
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q4k_gemv_ex(dev(w3), dev(x3), y3, n, 8192, 5, kernel=4)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    w4, x4 = synth.make_inputs(n, 18432, 2, seed=8)
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q4k_gemv_ex(dev(w4), dev(x4), y3, n, 18432, 2, kernel=4)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.count_nonzero(y3).item() == 0
    torch.cuda.synchronize()
    assert torch.count_nonzero(y_d).item() == 0


def _x_cases(rng, k):
    """x with wide dynamic range: outliers, tiny and zero columns, mixed
    magnitudes across 256-element columns, subnormal f32 values."""
    base = rng.standard_normal(k)
    out = base.copy()
    out[::97] *= 1e4                       # outliers
    out[256:512] = 0.0                     # an all-zero column
    if k >= 1024:
        out[512:768] *= 1e-30              # tiny column
        out[768:1024] *= 1e25              # huge column
    out[5] = 1e-40                         # f32 subnormal
    out[7] = -3e-39
    return np.stack([base, out]).astype(np.float32)


@pytest.mark.parametrize("n,k", [(64, 2048), (33, 4096)])
def test_lines_kernel_x_dynamic_range(oracle_mod, n, k):
    rng = np.random.default_rng(n * k)
    w, _ = synth.make_inputs(n, k, 1, seed=n + k)
    xs = _x_cases(rng, k)
    w_d = dev(w)
    for b in range(xs.shape[0]):
        x = xs[b:b + 1]
        y_ref, bound = oracle_mod.gemv(w, x, n)
        for opts in LINES_VARIANTS[:2]:
            _say("matrix-core dynamic range n=%d k=%d case %d %r" % (n, k, b, opts))
            y = run_gemv(w_d, x, n, k, 1, **opts)
            assert_within(y, y_ref, bound, "matrix-core x case %d %r" % (b, opts))


@pytest.mark.parametrize("i", [0, 1, 2])
def test_variants_bit_identical(oracle_mod, i):
    wl, w, x, y_ref, bound = workload(i, oracle_mod)
    w_d = dev(w)
    base = run_gemv(w_d, x, wl.n, wl.k, wl.m, kernel=1)
    assert_within(base, y_ref, bound, "x-stager kernel")
    for opts in VARIANTS:
        _say("workload %d variant %r" % (i, opts))
        try:
            y = run_gemv(w_d, x, wl.n, wl.k, wl.m, **opts)
        except q4k.Q4KError as e:
            if e.rc == q4k.Q4K_ERR_UNSUPPORTED:      # e.g. x in registers needs one span
                _say("  not applicable to this shape")
                continue
            raise
        assert np.array_equal(y.view(np.uint32), base.view(np.uint32)), opts


@pytest.mark.parametrize("m", range(1, 9))
def test_batched_equals_separate_calls(oracle_mod, m):
    n, k = 300, 4096 + 1024   # two spans, the second ragged
    w, x = synth.make_inputs(n, k, m, seed=77 + m)
    _say("batched m=%d n=%d k=%d" % (m, n, k))
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    yauto = run_gemv(w_d, x, n, k, m)
    assert_within(yauto, y_ref, bound, "batched m=%d" % m)
    yb = run_gemv(w_d, x, n, k, m, kernel=1)
    assert_within(yb, y_ref, bound, "batched m=%d, x-stager kernel" % m)
    for b in range(m):
        # the same kernel family at m = 1 is bit-identical; the default m = 1
        # kernel (streaming) reduces in another order and is within tolerance
        y1 = run_gemv(w_d, x[b:b + 1], n, k, 1, kernel=1)
        assert np.array_equal(y1[0].view(np.uint32), yb[b].view(np.uint32)), b
        y2 = run_gemv(w_d, x[b:b + 1], n, k, 1)
        assert_within(y2, y_ref[b:b + 1], bound[b:b + 1], "m=1 default, vector %d" % b)


def test_batched_workload_against_separate(oracle_mod):
    """The batched workload: the automatic kernel (sub-block, column window;
    its single-vector counterpart: per-wave x, the same sums) and the
    x-stager kernel, each bit-identical to m single-vector launches."""
    wl, w, x, y_ref, bound = workload(4, oracle_mod)
    w_d = dev(w)
    for opts, single in ((dict(), dict(kernel=6)), (dict(kernel=1), dict(kernel=1))):
        _say("batched workload 4 %r" % opts)
        yb = run_gemv(w_d, x, wl.n, wl.k, wl.m, **opts)
        assert_within(yb, y_ref, bound, "batched workload %r" % opts)
        for b in range(wl.m):
            y1 = run_gemv(w_d, x[b:b + 1], wl.n, wl.k, 1, **single)
            assert np.array_equal(y1[0].view(np.uint32), yb[b].view(np.uint32)), (opts, b)


EDGE_SHAPES = [
    (1, 256, 1), (3, 256, 1), (255, 512, 1), (257, 768, 1), (64, 4096 - 256, 1),
    (17, 4096 + 256, 1), (33, 5 * 4096 + 768, 1), (1, 65536, 1), (129, 256, 8),
    (7, 12288, 3), (9, 12288 + 256, 2), (40, 14336, 8), (5, 1024, 5),
]


@pytest.mark.parametrize("n,k,m", EDGE_SHAPES)
def test_edge_shapes(oracle_mod, n, k, m):
    _say("edge n=%d k=%d m=%d" % (n, k, m))
    w, x = synth.make_inputs(n, k, m, seed=n * 7919 + k + m)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    y = run_gemv(w_d, x, n, k, m)
    assert_within(y, y_ref, bound, "n=%d k=%d m=%d" % (n, k, m))
    out = torch.empty((n, k), dtype=torch.float32, device="cuda")
    q4k.q4k_dequantize(w_d, out, n, k)
    torch.cuda.synchronize()
    ref = oracle_mod.dequant(w, n, k)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_special_header_values(oracle_mod):
    """Signed zeros, subnormal, largest and negative d/dmin: dequant bit-exact,
    y within tolerance (finite cases)."""
    specials = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0xBC00, 0x3C00,
                         0x1234], np.uint16)
    rng = np.random.default_rng(31)
    n = specials.size * specials.size
    S = 2
    f = synth.draw_fields(rng, n, S)
    f.d_bits[:, 0] = np.repeat(specials, specials.size)
    f.dmin_bits[:, 0] = np.tile(specials, specials.size)
    f.d_bits[:, 1] = np.tile(specials, specials.size)
    f.dmin_bits[:, 1] = np.repeat(specials, specials.size)
    w = synth.pack(f)
    k = 256 * S
    x = rng.standard_normal((2, k)).astype(np.float32)
    w_d = dev(w)
    out = torch.empty((n, k), dtype=torch.float32, device="cuda")
    q4k.q4k_dequantize(w_d, out, n, k)
    torch.cuda.synchronize()
    ref = oracle_mod.dequant(w, n, k)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    y_ref, bound = oracle_mod.gemv(w, x, n)
    y = run_gemv(w_d, x, n, k, 2)
    assert_within(y, y_ref, bound, "special headers")


def test_zero_weights_and_zero_x(oracle_mod):
    n, k = 37, 2048
    rng = np.random.default_rng(8)
    f = synth.draw_fields(rng, n, k // 256)
    f.sc[:] = 0
    f.m[:] = 0
    w = synth.pack(f)
    x = rng.standard_normal((1, k)).astype(np.float32)
    y = run_gemv(dev(w), x, n, k, 1)
    assert np.all(y == 0)
    w2, _ = synth.make_inputs(n, k, 1, seed=3)
    y2 = run_gemv(dev(w2), np.zeros((1, k), np.float32), n, k, 1)
    assert np.all(y2 == 0)


def test_uniform_row_closed_form(oracle_mod):
    """Uniform q, sc, m, d, dmin give a constant row c, y = c * sum(x)."""
    n, S = 9, 20
    k = 256 * S
    f = synth.Fields(np.full((n, S), 0x2E66, np.uint16), np.full((n, S), 0x2A00, np.uint16),
                     np.full((n, S, 8), 37, np.uint8), np.full((n, S, 8), 12, np.uint8),
                     np.full((n, S, 256), 9, np.uint8))
    w = synth.pack(f)
    rng = np.random.default_rng(10)
    x = rng.standard_normal((1, k)).astype(np.float32)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    y = run_gemv(dev(w), x, n, k, 1)
    assert_within(y, y_ref, bound, "uniform rows")
    assert np.all(y == y[0, 0])


def test_quantized_real_valued_rows(oracle_mod):
    """Rows produced by the reference quantizer from N(0,1) data (realistic
    scale/min structure rather than independent uniform fields)."""
    rng = np.random.default_rng(44)
    n, k = 128, 4096
    src = rng.standard_normal((n, k)).astype(np.float32)
    w = oracle_mod.quantize_rows(src)
    x = rng.standard_normal((3, k)).astype(np.float32)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    y = run_gemv(dev(w), x, n, k, 3)
    assert_within(y, y_ref, bound, "quantized rows")


def test_nonzero_stream_and_overwrite(oracle_mod):
    wl, w, x, y_ref, bound = workload(0, oracle_mod)
    s = torch.cuda.Stream()
    w_d = dev(w)
    x_d = dev(x)
    y_d = torch.full((wl.m, wl.n), 123.0, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        q4k.q4k_gemv(w_d, x_d, y_d, wl.n, wl.k, wl.m, stream=s)
    s.synchronize()
    assert_within(y_d.cpu().numpy(), y_ref, bound, "side stream")


def test_plan_query_on_device():
    """q4k_plan asking the device for its LDS size plans as it does with
    gfx950's 160 KiB given explicitly."""
    for shp in [(32000, 4096, 1), (4096, 14336, 1), (4096, 4096, 1), (14336, 4096, 8),
                (4096, 14336, 8), (32000, 4096, 2)]:
        a = q4k.q4k_plan(*shp, lds_max=0)
        b = q4k.q4k_plan(*shp, lds_max=163840)
        assert [getattr(a, f) for f, _ in a._fields_] == [getattr(b, f) for f, _ in b._fields_]


def _random_cases(count, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        m = int(rng.choice([1, 1, 1, 2, 3, 4, 5, 6, 7, 8]))
        if m == 1 and rng.random() < 0.5:
            n = int(rng.integers(2000, 9000))
            S = int(rng.choice([16, 24, 32, 40, 43, 56]))
        else:
            n = int(rng.integers(1, 1500))
            S = int(rng.integers(1, 80))
        off = int(rng.choice([0, 0, 16, 48]))
        cases.append((n, 256 * S, m, off))
    return cases


@pytest.mark.parametrize("n,k,m,off", _random_cases(24, 2026))
def test_random_shapes_automatic_plan(oracle_mod, n, k, m, off):
    """Seeded random shapes, batch sizes and weight-buffer offsets (16-byte
    aligned, not always 128-byte aligned) through q4k_gemv's automatic plan."""
    p = q4k.q4k_plan(n, k, m, w_aligned128=(off == 0))
    _say("random n=%d k=%d m=%d off=%d -> kernel %d" % (n, k, m, off, p.kernel))
    if off:
        assert p.kernel <= 2   # the line-streamed kernels need 128-byte aligned rows
    w, x = synth.make_inputs(n, k, m, seed=n * 131 + k + m)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    buf = torch.empty(w.size + off, dtype=torch.uint8, device="cuda")
    buf[off:].copy_(torch.from_numpy(w))
    w_d = buf[off:]
    assert w_d.data_ptr() % 128 == off % 128
    y = run_gemv(w_d, x, n, k, m)
    assert_within(y, y_ref, bound, "n=%d k=%d m=%d off=%d" % (n, k, m, off))


# 9-32 vectors: one pass over the weights for up to eight quads of vectors on
# the sub-block kernels (beyond four quads: kernel 6 only).  Per vector the
# digits, MFMAs and sums are those of a single-vector launch of the same
# kernel and column grouping.
@pytest.mark.parametrize("n,k,m", [(300, 4096, 16), (130, 4096, 9), (17, 2048, 12), (64, 8192, 13),
                                   (33, 2048, 15), (1, 2048, 10), (257, 16384, 16),
                                   (40, 14336, 11),
                                   # rows of partial slabs: kernel 5's whole x stage
                                   (17, 1280, 13), (5, 768, 16), (70, 1536, 9),
                                   # five to eight quads
                                   (300, 4096, 32), (17, 1280, 17), (64, 8192, 24),
                                   (40, 14336, 32), (5, 768, 20), (1, 2048, 29), (130, 11008, 27)])
def test_wide_batch(oracle_mod, n, k, m):
    w, x = synth.make_inputs(n, k, m, seed=n * 37 + k + 11 * m)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    _say("wide batch n=%d k=%d m=%d" % (n, k, m))
    y = run_gemv(w_d, x, n, k, m)               # automatic kernel
    assert_within(y, y_ref, bound, "wide batch automatic m=%d" % m)
    ran = []
    for kern in (5, 6):
        try:
            yk = run_gemv(w_d, x, n, k, m, kernel=kern, cols_per_task=8)
        except q4k.Q4KError as e:
            assert e.rc == q4k.Q4K_ERR_UNSUPPORTED
            continue
        ran.append(kern)
        assert_within(yk, y_ref, bound, "wide batch kernel %d m=%d" % (kern, m))
        for b in range(m):                      # batched == m single-vector launches
            y1 = run_gemv(w_d, x[b:b + 1], n, k, 1, kernel=kern, cols_per_task=8)
            assert np.array_equal(y1[0].view(np.uint32), yk[b].view(np.uint32)), (kern, b)
    assert ran


def test_wide_batch_full_size(oracle_mod):
    """14336 x 4096 with sixteen vectors (automatic: one pass on kernel 7)
    against the oracle, and against two calls of eight vectors on the same
    kernel and column grouping (bit-identical)."""
    n, k, m = 14336, 4096, 16
    w, x = synth.make_inputs(n, k, m, seed=14336 + 4096 + 16)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    _say("wide batch automatic n=%d k=%d m=%d" % (n, k, m))
    assert q4k.q4k_plan(n, k, m).kernel == 7
    y = run_gemv(w_d, x, n, k, m)
    assert_within(y, y_ref, bound, "14336 x 4096 m=16")
    y16 = run_gemv(w_d, x, n, k, m, kernel=6, cols_per_task=8)
    assert_within(y16, y_ref, bound, "14336 x 4096 m=16 one pass")
    assert np.array_equal(y16.view(np.uint32), y.view(np.uint32))
    for h in range(2):
        y8 = run_gemv(w_d, x[8 * h:8 * h + 8], n, k, 8, kernel=6, cols_per_task=8)
        assert np.array_equal(y8.view(np.uint32), y16[8 * h:8 * h + 8].view(np.uint32)), h


def test_wide_batch_32_full_size(oracle_mod):
    """14336 x 4096 with 32 vectors (automatic: kernel 6 on eight quads, one
    pass over the weights) against the oracle, and against two calls of
    sixteen vectors on the same kernel and column grouping (bit-identical)."""
    n, k, m = 14336, 4096, 32
    w, x = synth.make_inputs(n, k, m, seed=14336 + 4096 + 32)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    w_d = dev(w)
    _say("wide batch automatic n=%d k=%d m=%d" % (n, k, m))
    p = q4k.q4k_plan(n, k, m)
    assert p.kernel == 6 and p.threads == 256
    y = run_gemv(w_d, x, n, k, m)
    assert_within(y, y_ref, bound, "14336 x 4096 m=32")
    for h in range(2):
        y16 = run_gemv(w_d, x[16 * h:16 * h + 16], n, k, 16, kernel=6,
                       cols_per_task=p.cols_per_task)
        assert np.array_equal(y16.view(np.uint32), y[16 * h:16 * h + 16].view(np.uint32)), h


@pytest.mark.parametrize("n,k,m,off", [(300, 4096, 12, 0), (130, 11008, 16, 0), (33, 2304, 9, 48),
                                       (4096, 14336, 16, 0), (4096, 14336, 32, 0),
                                       (33, 2304, 20, 48)])
def test_wide_batch_automatic(oracle_mod, n, k, m, off):
    """Automatic plans of 9-16 vectors: one pass against the oracle, or a
    refusal (unaligned weights; rows whose sixteen-vector plan exceeds the
    LDS) that launches nothing and leaves y untouched."""
    w, x = synth.make_inputs(n, k, m, seed=n * 41 + k + 13 * m)
    buf = torch.empty(w.size + off, dtype=torch.uint8, device="cuda")
    buf[off:].copy_(torch.from_numpy(w))
    w_d = buf[off:]
    try:
        p = q4k.q4k_plan(n, k, m, w_aligned128=(off == 0))
    except q4k.Q4KError as e:
        assert e.rc == q4k.Q4K_ERR_UNSUPPORTED
        _say("wide batch automatic n=%d k=%d m=%d off=%d -> refused" % (n, k, m, off))
        x_d = dev(x)
        y_d = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda")
        with pytest.raises(q4k.Q4KError) as ei:
            q4k.q4k_gemv(w_d, x_d, y_d, n, k, m)
        assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        assert bool((y_d == 7.0).all())
        return
    _say("wide batch automatic n=%d k=%d m=%d off=%d -> kernel %d" % (n, k, m, off, p.kernel))
    assert p.kernel in (5, 6, 7)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    y = run_gemv(w_d, x, n, k, m)
    assert_within(y, y_ref, bound, "n=%d k=%d m=%d off=%d" % (n, k, m, off))

"""The C-ABI library on the CPU: it loads, exports every symbol include/q4k.h
declares, and refuses bad arguments with the documented status before any
HIP call (so none of these calls touches a device).

The refusal cases follow the pages' own validation tests (turbospark-runtime
0.1.0, real_forward_dispatch.rs, test module: valid shape, wrong shape, a byte
count short by one block) and the pre-launch pointer checks of realizar 0.8.5
(q4k_gemv_cached.rs: `q4k_gemv_indexed_async`).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from block_quantized_decode_q4_amd import q4k

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4k.h")

A = 0x100000          # a 16-byte-aligned fake device address (never dereferenced)
MIS = 0x100004        # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4k_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return q4k.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(q4k.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for rc in (0, 1, 2, 3, 4, 5, 1001, 77):
        s = q4k.status_string(rc)
        assert isinstance(s, str) and s
    assert q4k.status_string(0) == "ok"


def test_row_bytes():
    assert q4k.q4k_row_bytes(256) == 144
    assert q4k.q4k_row_bytes(4096) == 16 * 144
    assert q4k.q4k_row_bytes(14336) == 56 * 144
    for bad in (0, -256, 255, 257, 100):
        assert q4k.q4k_row_bytes(bad) == 0


def raw_gemv(lib, w, x, y, n, k, m):
    return lib.q4k_gemv(w, x, y, n, k, m, None)


def test_gemv_refusals(lib):
    assert raw_gemv(lib, None, A, A, 16, 256, 1) == q4k.Q4K_ERR_NULL
    assert raw_gemv(lib, A, None, A, 16, 256, 1) == q4k.Q4K_ERR_NULL
    assert raw_gemv(lib, A, A, None, 16, 256, 1) == q4k.Q4K_ERR_NULL
    for n, k, m in ((0, 256, 1), (-1, 256, 1), (16, 255, 1), (16, 0, 1), (16, 384, 1),
                    (16, 256, 0), (16, 256, -3), (2 ** 31, 256, 1), (16, 2 ** 31 + 256, 1)):
        assert raw_gemv(lib, A, A, A, n, k, m) == q4k.Q4K_ERR_SHAPE, (n, k, m)
    for m in (17, 32):
        assert raw_gemv(lib, A, A, A, 16, 256, m) == q4k.Q4K_ERR_UNSUPPORTED
    assert raw_gemv(lib, MIS, A, A, 16, 256, 1) == q4k.Q4K_ERR_ALIGN
    assert raw_gemv(lib, A, MIS, A, 16, 256, 1) == q4k.Q4K_ERR_ALIGN
    assert raw_gemv(lib, A, A, MIS, 16, 256, 1) == q4k.Q4K_ERR_ALIGN


def test_gemv_ex_refusals(lib):
    bad_opts = [dict(variant=3), dict(variant=-1), dict(waves_per_block=2), dict(rows_per_wave=3),
                dict(x_in_registers=5)]
    for o in bad_opts:
        cfg = q4k.q4k_launch(**o)
        rc = lib.q4k_gemv_ex(A, A, A, 16, 256, 1, ctypes.byref(cfg), None)
        assert rc == q4k.Q4K_ERR_UNSUPPORTED, o
    # x in registers needs one span and one vector
    cfg = q4k.q4k_launch(x_in_registers=1)
    assert lib.q4k_gemv_ex(A, A, A, 16, 8192, 1, ctypes.byref(cfg), None) == q4k.Q4K_ERR_UNSUPPORTED
    assert lib.q4k_gemv_ex(A, A, A, 16, 256, 2, ctypes.byref(cfg), None) == q4k.Q4K_ERR_UNSUPPORTED
    # four rows per wave only for one vector
    cfg = q4k.q4k_launch(rows_per_wave=4)
    assert lib.q4k_gemv_ex(A, A, A, 16, 256, 2, ctypes.byref(cfg), None) == q4k.Q4K_ERR_UNSUPPORTED


def test_launch_struct_matches_header():
    """The binding's q4k_launch has the fields of the C struct, in order,
    all int32."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    body = re.search(r"typedef struct q4k_launch \{(.*?)\} q4k_launch;", text, re.S).group(1)
    fields = re.findall(r"int32_t\s+([a-z_0-9]+)\s*;", body)
    assert fields == [f for f, _ in q4k.q4k_launch._fields_]
    assert all(t is ctypes.c_int32 for _, t in q4k.q4k_launch._fields_)
    assert ctypes.sizeof(q4k.q4k_launch) == 4 * len(fields)


def test_gemv_ex_kernel_option_refusals(lib):
    """Options that no kernel can honour are refused before any HIP call."""
    cases = [
        (dict(kernel=7), 16, 2048, 1),                       # kernels 1-6 only
        (dict(kernel=-1), 16, 2048, 1),
        (dict(kernel=2), 16, 2048, 2),                       # streaming: one vector
        (dict(kernel=3), 16, 4096, 2),                       # vector-ALU lines: one vector
        (dict(kernel=3, ring_depth=9), 16, 1024, 1),         # partial slabs: three lines
        (dict(kernel=3, waves_per_block=16, ring_depth=9), 16, 4096, 1),
        (dict(kernel=3, waves_per_block=8), 16, 65536, 1),   # x: four groups per lane at most
        (dict(kernel=3, ring_depth=4), 16, 4096, 1),
        (dict(kernel=4), 16, 1024, 1),                       # k not a multiple of 2048
        (dict(kernel=4, cols_per_task=12), 16, 4096, 1),     # whole slabs only
        (dict(kernel=4, cols_per_task=24), 16, 4096, 1),     # must divide the row's slabs
        (dict(kernel=4, ring_depth=4), 16, 4096, 1),
        (dict(kernel=4, waves_per_block=16, ring_depth=9), 16, 4096, 1),
        (dict(kernel=4, waves_per_block=4), 16, 4096, 2),    # several vectors: 8 waves
        (dict(kernel=4, rows_per_task=2), 16, 4096, 1),
        (dict(kernel=5, waves_per_block=4), 16, 4096, 2),    # eight waves only
        (dict(kernel=5, ring_depth=9), 16, 4096, 2),         # three lines in flight only
        (dict(kernel=6, waves_per_block=16), 16, 4096, 2),   # eight waves only
        (dict(kernel=6, ring_depth=9), 16, 4096, 8),         # three lines in flight only
        (dict(kernel=1, cols_per_task=8), 16, 4096, 1),      # line-streamed options only
        (dict(kernel=2, cols_per_task=8), 16, 4096, 1),
    ]
    for o, n, k, m in cases:
        cfg = q4k.q4k_launch(**o)
        rc = lib.q4k_gemv_ex(A, A, A, n, k, m, ctypes.byref(cfg), None)
        assert rc == q4k.Q4K_ERR_UNSUPPORTED, (o, n, k, m, rc)


def test_load_refusals(lib):
    host = np.zeros(4 * 144 * 2, np.uint8)
    hp = host.ctypes.data
    assert lib.q4k_load(None, hp, host.nbytes, 2, 1024, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_load(A, None, host.nbytes, 2, 1024, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_load(A, hp, host.nbytes, 2, 1000, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_load(A, hp, host.nbytes - 144, 2, 1024, None) == q4k.Q4K_ERR_SIZE   # short by one block
    assert lib.q4k_load(A, hp, host.nbytes + 1, 2, 1024, None) == q4k.Q4K_ERR_SIZE
    assert lib.q4k_load(A, hp, host.nbytes, 3, 1024, None) == q4k.Q4K_ERR_SIZE           # wrong row count
    assert lib.q4k_load(MIS, hp, host.nbytes, 2, 1024, None) == q4k.Q4K_ERR_ALIGN


def test_dequant_and_calibrate_refusals(lib):
    assert lib.q4k_dequantize(None, A, 4, 256, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_dequantize(A, None, 4, 256, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_dequantize(A, A, 4, 300, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_dequantize(A, A, 0, 256, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_dequantize(A, MIS, 4, 256, None) == q4k.Q4K_ERR_ALIGN
    assert lib.q4k_read_calibrate(None, 16, A, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_read_calibrate(A, 20, A, None) == q4k.Q4K_ERR_SIZE
    assert lib.q4k_read_calibrate(A, 0, A, None) == q4k.Q4K_ERR_SIZE
    assert lib.q4k_read_calibrate(MIS, 32, A, None) == q4k.Q4K_ERR_ALIGN
    assert q4k.q4k_read_calibrate_blocks() > 0


def test_binding_raises_with_status():
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_gemv(0, A, A, 16, 256, 1, stream=0)
    assert ei.value.rc == q4k.Q4K_ERR_NULL
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_gemv(A, A, A, 16, 256, 17, stream=0)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED


MI355X_LDS = 163840   # LDS bytes per workgroup on gfx950


def test_plan_info_struct_matches_header():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    body = re.search(r"typedef struct q4k_plan_info \{(.*?)\} q4k_plan_info;", text, re.S).group(1)
    fields = re.findall(r"int32_t\s+([a-z_0-9]+)\s*;", body)
    assert fields == [f for f, _ in q4k.q4k_plan_info._fields_]
    assert all(t is ctypes.c_int32 for _, t in q4k.q4k_plan_info._fields_)


@pytest.mark.parametrize("n,k,m,aligned,kernel,grid,cols", [
    (32000, 4096, 1, True, 3, 250, 16),     # LM head: 64 MiB of weights, 128 rows a block
    (4096, 14336, 1, True, 3, 256, 8),      # FFN down: 16 rows a block, slab tasks
    (16384, 16384, 1, True, 3, 256, 8),
    (4096, 4096, 1, True, 2, 256, 0),       # 9 MiB: below the line-stream threshold
    (256, 1024, 1, True, 2, 32, 0),
    (32000, 4096, 1, False, 2, None, 0),    # weights not 128-byte aligned
    (32000, 4096, 2, True, 4, 250, 16),     # m = 2: line MFMA
    (14336, 4096, 8, True, 5, 224, 8),      # m >= 3: sub-block MFMA, x staged whole
    (4096, 14336, 8, True, 6, 256, 8),      # x of 8 columns does not fit: per-wave x
    (4096, 11008, 8, True, 6, 256, 8),      # partial slab (43 superblocks)
    (14336, 4096, 8, False, 1, None, 0),
])
def test_plan_automatic_choice(n, k, m, aligned, kernel, grid, cols):
    """The automatic rule of q4k_gemv_ex, asked without a GPU."""
    p = q4k.q4k_plan(n, k, m, w_aligned128=aligned, lds_max=MI355X_LDS)
    assert p.kernel == kernel
    if grid is not None:
        assert p.grid == grid
    assert p.cols_per_task == cols
    assert p.threads % 64 == 0 and 64 <= p.threads <= 1024
    assert 0 < p.lds_bytes <= MI355X_LDS
    assert p.grid * p.rows_per_block >= n
    assert (p.grid - 1) * p.rows_per_block < n
    if kernel <= 2:
        assert p.spans_per_chunk >= 1
    else:
        assert p.spans_per_chunk == 0 and p.ring_depth == 3


def test_plan_follows_options_and_lds_limit():
    p = q4k.q4k_plan(32000, 4096, 1, lds_max=MI355X_LDS, kernel=4)
    assert p.kernel == 4
    p = q4k.q4k_plan(32000, 4096, 1, lds_max=MI355X_LDS, kernel=3, cols_per_task=8)
    assert p.kernel == 3 and p.cols_per_task == 8
    # the whole-x stage of kernel 5 (150848 bytes here) does not fit in 64 KiB:
    # the automatic choice moves on to per-wave x
    p = q4k.q4k_plan(14336, 4096, 8, lds_max=MI355X_LDS)
    assert p.kernel == 5 and p.lds_bytes == 150848
    p = q4k.q4k_plan(14336, 4096, 4, lds_max=65536)
    assert p.kernel == 6 and p.lds_bytes <= 65536
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_plan(14336, 4096, 8, lds_max=65536, kernel=5)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED


def test_plan_refusals(lib):
    out = q4k.q4k_plan_info()
    assert lib.q4k_plan(4096, 4096, 1, None, 1, MI355X_LDS, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_plan(16, 100, 1, None, 1, MI355X_LDS, ctypes.byref(out)) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_plan(16, 256, 17, None, 1, MI355X_LDS, ctypes.byref(out)) == q4k.Q4K_ERR_UNSUPPORTED
    assert lib.q4k_plan(16, 256, 9, None, 0, MI355X_LDS, ctypes.byref(out)) == q4k.Q4K_OK
    assert out.launches == 2 and out.kernel == 1     # unaligned: two x-stager launches
    cfg = q4k.q4k_launch(kernel=3)
    assert lib.q4k_plan(32000, 4096, 2, ctypes.byref(cfg), 1, MI355X_LDS,
                        ctypes.byref(out)) == q4k.Q4K_ERR_UNSUPPORTED


@pytest.mark.parametrize("n,k,m,aligned,launches,kernel", [
    (4096, 14336, 16, True, 1, 6),     # eight vectors take kernel 6 too: one pass
    (300, 2048, 12, True, 1, 5),       # sixteen vectors' x fits one stage
    (17, 1280, 13, True, 1, 5),        # partial slab, whole stage
    (5, 256, 16, True, 1, 5),
    (14336, 4096, 16, True, 2, 5),     # eight vectors stage x whole: two launches
    (14336, 4096, 9, True, 2, 5),
    (32000, 4096, 16, True, 2, 5),
    (130, 11008, 16, True, 2, 6),      # sixteen vectors' plan exceeds the LDS
    (14336, 4096, 9, False, 2, 1),     # weights not 128-byte aligned
])
def test_plan_wide_batches(n, k, m, aligned, launches, kernel):
    """9-16 vectors: one pass over the weights, or two launches of at most
    eight vectors (the fields describe the first)."""
    p = q4k.q4k_plan(n, k, m, w_aligned128=aligned, lds_max=MI355X_LDS)
    assert (p.launches, p.kernel) == (launches, kernel)
    assert p.lds_bytes <= MI355X_LDS
    if launches == 2:
        first = q4k.q4k_plan(n, k, 8, w_aligned128=aligned, lds_max=MI355X_LDS)
        assert [getattr(p, f) for f, _ in p._fields_][:-1] == \
            [getattr(first, f) for f, _ in first._fields_][:-1]
    for m1 in range(1, 9):
        assert q4k.q4k_plan(n, k, m1, w_aligned128=aligned, lds_max=MI355X_LDS).launches == 1


def test_plan_wide_batch_refusals():
    for opts in (dict(kernel=1), dict(kernel=4), dict(rows_per_block=64)):
        with pytest.raises(q4k.Q4KError) as ei:
            q4k.q4k_plan(14336, 4096, 9, lds_max=MI355X_LDS, **opts)
        assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    # rows of partial slabs whose x of 16 vectors does not fit one stage:
    # kernel 6's four-line rings and four quads exceed the LDS
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_plan(130, 11008, 16, lds_max=MI355X_LDS, kernel=6)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    # a forced kernel is one launch
    p = q4k.q4k_plan(14336, 4096, 16, lds_max=MI355X_LDS, kernel=6)
    assert (p.launches, p.kernel) == (1, 6)

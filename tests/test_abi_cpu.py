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
    return sorted(set(re.findall(r"\b(q[46]k_[a-z0-9_]+)\s*\(", text)))


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
    for m in (33, 64):
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
        (dict(kernel=8), 16, 2048, 1),                       # kernels 1-7 only
        (dict(kernel=7), 16, 1280, 2),                       # window: whole slabs only
        (dict(kernel=7, ring_depth=9), 16, 4096, 8),         # three lines in flight only
        (dict(kernel=7, rows_per_block=80), 16, 4096, 8),    # 5 tiles x 2 slabs > 8 waves
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
        q4k.q4k_gemv(A, A, A, 16, 256, 33, stream=0)
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
    (14336, 4096, 4, True, 5, 224, 8),      # m >= 3: sub-block MFMA, x staged whole
    (14336, 4096, 8, True, 7, 224, 8),      # x of 8 vectors does not fit one stage: window
    (14336, 8192, 8, True, 7, 448, 8),      # four slabs: 32 rows a workgroup
    (4096, 14336, 8, True, 6, 256, 8),      # 7 slabs x 2 quads: no window; per-wave x
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
    # the whole-x stage of kernel 5 for eight vectors (33 groups of 4752
    # bytes and eight rings of 4352) exceeds the LDS: the automatic choice
    # moves on to the column window (two columns of each of two slabs for
    # two quads; eight rings; f64 row sums of two slab groups of 64 rows)
    p = q4k.q4k_plan(14336, 4096, 8, lds_max=MI355X_LDS)
    assert p.kernel == 7 and p.lds_bytes == 2 * 2 * 2 * 4752 + 8 * 4352 + 2 * 64 * 8 * 8
    assert p.rows_per_block == 64 and p.cols_per_task == 8
    # per-wave x: one group's digits and constants (4608 bytes) and two
    # quads' lists (144 each) per wave
    p = q4k.q4k_plan(14336, 4096, 8, lds_max=MI355X_LDS, kernel=6)
    assert p.lds_bytes == 8 * (4608 + 2 * 144) + 8 * 4352 + 2 * 64 * 8 * 8
    # four vectors: 17 groups and the rings fit 160 KiB, not 96 KiB
    p = q4k.q4k_plan(14336, 4096, 4, lds_max=MI355X_LDS)
    assert p.kernel == 5
    p = q4k.q4k_plan(14336, 4096, 4, lds_max=98304)
    assert p.kernel == 7 and p.lds_bytes <= 98304
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_plan(14336, 4096, 8, lds_max=MI355X_LDS, kernel=5)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED


def test_plan_refusals(lib):
    out = q4k.q4k_plan_info()
    assert lib.q4k_plan(4096, 4096, 1, None, 1, MI355X_LDS, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_plan(16, 100, 1, None, 1, MI355X_LDS, ctypes.byref(out)) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_plan(16, 256, 33, None, 1, MI355X_LDS, ctypes.byref(out)) == q4k.Q4K_ERR_UNSUPPORTED
    # 9-32 vectors need the one-pass sub-block kernels, which need 128-byte
    # aligned weights: refused, never split into two launches
    assert lib.q4k_plan(16, 256, 9, None, 0, MI355X_LDS, ctypes.byref(out)) == \
        q4k.Q4K_ERR_UNSUPPORTED
    cfg = q4k.q4k_launch(kernel=3)
    assert lib.q4k_plan(32000, 4096, 2, ctypes.byref(cfg), 1, MI355X_LDS,
                        ctypes.byref(out)) == q4k.Q4K_ERR_UNSUPPORTED


@pytest.mark.parametrize("n,k,m,kernel", [
    (4096, 14336, 16, 6),     # x per column per wave
    (300, 2048, 12, 7),       # one slab x four quads: the window
    (17, 1280, 13, 6),        # partial slabs
    (130, 11008, 16, 6),
    (5, 256, 16, 5),          # sixteen vectors' x fits one stage
    (3, 768, 9, 5),
    (14336, 4096, 16, 7),     # two slabs x four quads: the window
    (14336, 4096, 9, 7),
    (32000, 4096, 16, 7),
    (14336, 8192, 16, 6),     # four slabs x four quads: per-wave x
    (14336, 4096, 32, 6),     # five to eight quads: per-wave x only
    (4096, 14336, 32, 6),
    (17, 1280, 17, 6),
    (32000, 4096, 24, 6),
])
def test_plan_wide_batches(n, k, m, kernel):
    """9-32 vectors: one pass over the weights on a sub-block kernel."""
    p = q4k.q4k_plan(n, k, m, lds_max=MI355X_LDS)
    assert p.kernel == kernel
    assert p.lds_bytes <= MI355X_LDS


@pytest.mark.parametrize("n,k,m,aligned", [
    (14336, 4096, 9, False),  # weights not 128-byte aligned
    (64, 4096, 12, False),
    (14336, 4096, 32, False),
])
def test_plan_wide_batches_refused(n, k, m, aligned):
    """9-32 vectors where no one-pass kernel applies: refused by name, not
    split into launches of at most eight (turbospark-runtime 0.1.0,
    real_forward_dispatch.rs: doc of `encode_gemm_any`); eight still run."""
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_plan(n, k, m, w_aligned128=aligned, lds_max=MI355X_LDS)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    q4k.q4k_plan(n, k, 8, w_aligned128=aligned, lds_max=MI355X_LDS)


def test_plan_wide_batch_refusals():
    for opts in (dict(kernel=1), dict(kernel=4), dict(rows_per_block=64)):
        with pytest.raises(q4k.Q4KError) as ei:
            q4k.q4k_plan(14336, 4096, 9, lds_max=MI355X_LDS, **opts)
        assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    # more than sixteen vectors: kernel 6 only (eight quads of x do not fit
    # kernel 5's stage or kernel 7's window)
    for kern in (5, 7, 1, 4):
        with pytest.raises(q4k.Q4KError) as ei:
            q4k.q4k_plan(14336, 4096, 20, lds_max=MI355X_LDS, kernel=kern)
        assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    p = q4k.q4k_plan(14336, 4096, 32, lds_max=MI355X_LDS, kernel=6)
    assert p.kernel == 6 and p.threads == 256
    # kernel 6 with more than eight vectors runs four waves only
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_plan(14336, 4096, 16, lds_max=MI355X_LDS, kernel=6, waves_per_block=8)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    p = q4k.q4k_plan(14336, 4096, 16, lds_max=MI355X_LDS, kernel=6)
    assert p.kernel == 6 and p.threads == 256
    p = q4k.q4k_plan(14336, 4096, 8, lds_max=MI355X_LDS, kernel=6)
    assert p.threads == 512


@pytest.mark.parametrize("n,k,m,opts", [
    (300, 1280, 4, {}),                        # partial slab: no window
    (4096, 14336, 8, {}),                      # 7 slabs x 2 quads > 8 waves
    (4096, 20480, 1, {}),                      # 10 slabs > 8 waves
    (14336, 4096, 8, dict(rows_per_block=80)),  # 5 tiles x 2 slabs > 8 tasks
    (14336, 4096, 8, dict(cols_per_task=16)),  # one slab per task only
    (14336, 4096, 8, dict(waves_per_block=4)),
])
def test_plan_window_refusals(n, k, m, opts):
    """Kernel 7 (the workgroup's column window) only where every wave has at
    most one task of one slab and one window pair: anything else would make
    a wave meet the others' barriers a different number of times."""
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.q4k_plan(n, k, m, lds_max=MI355X_LDS, kernel=7, **opts)
    assert ei.value.rc == q4k.Q4K_ERR_UNSUPPORTED


@pytest.mark.parametrize("n,k,m,rpb", [(14336, 4096, 8, 64), (300, 4096, 3, 64), (33, 2048, 2, 128),
                                       (1, 16384, 1, 16), (14336, 4096, 16, 64), (64, 8192, 5, 32)])
def test_plan_window(n, k, m, rpb):
    p = q4k.q4k_plan(n, k, m, lds_max=MI355X_LDS, kernel=7)
    assert p.kernel == 7 and p.cols_per_task == 8 and p.threads == 512
    assert p.rows_per_block == rpb
    assert (rpb + 15) // 16 * (k // 2048) <= 8


def test_q8_refusals(lib):
    """The Q8 variant's argument checks, before any HIP call."""
    assert lib.q4k_gemv_q8(None, A, A, 16, 256, 1, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_gemv_q8(A, A, A, 16, 300, 1, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_gemv_q8(A, A, A, 0, 256, 1, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_gemv_q8(A, A, A, 16, 256, 0, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_gemv_q8(A, A, A, 16, 256, 2, None) == q4k.Q4K_ERR_UNSUPPORTED   # one vector
    assert lib.q4k_gemv_q8(A, MIS, A, 16, 256, 1, None) == q4k.Q4K_ERR_ALIGN
    assert lib.q4k_gemv_q8(A + 16, A, A, 16, 256, 1, None) == q4k.Q4K_ERR_UNSUPPORTED  # not 128-B aligned
    assert lib.q4k_quantize_q8(None, A, A, 64, 1, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_quantize_q8(A, A, A, 48, 1, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_quantize_q8(A, A, A, 0, 1, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_quantize_q8(A, A, A, 64, 0, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_quantize_q8(A, A, MIS, 64, 1, None) == q4k.Q4K_ERR_ALIGN


# ------------------------------------------------------------------ Q6_K
def test_q6k_row_bytes():
    assert q4k.q6k_row_bytes(256) == 210
    assert q4k.q6k_row_bytes(4096) == 16 * 210
    assert q4k.q6k_row_bytes(14336) == 56 * 210
    for bad in (0, -256, 255, 257):
        assert q4k.q6k_row_bytes(bad) == 0


def test_q6k_structs_match_header():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    for name, cls in (("q6k_launch", q4k.q6k_launch), ("q6k_plan_info", q4k.q6k_plan_info)):
        body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, re.S).group(1)
        fields = re.findall(r"int32_t\s+([a-z_0-9]+)\s*;", body)
        assert fields == [f for f, _ in cls._fields_], name
        assert all(t is ctypes.c_int32 for _, t in cls._fields_)


def test_q6k_refusals(lib):
    """Argument checks of the Q6_K entry points, before any HIP call."""
    g = lib.q6k_gemv
    assert g(None, A, A, 16, 4096, 0, None) == q4k.Q4K_ERR_NULL
    assert g(A, None, A, 16, 4096, 0, None) == q4k.Q4K_ERR_NULL
    assert g(A, A, None, 16, 4096, 0, None) == q4k.Q4K_ERR_NULL
    for n, k in ((0, 2048), (16, 300), (16, 0), (2 ** 31, 2048)):
        assert g(A, A, A, n, k, 0, None) == q4k.Q4K_ERR_SHAPE, (n, k)
    assert g(A, A, A, 16, 2048, 1679, None) == q4k.Q4K_ERR_SHAPE       # below the row's bytes
    assert g(A, A, A, 16, 2048, 1688, None) == q4k.Q4K_ERR_ALIGN       # not a multiple of 16
    assert g(A, A, A, 16, 1024, 0, None) == q4k.Q4K_ERR_ALIGN          # dense 840-byte rows
    assert g(MIS, A, A, 16, 2048, 0, None) == q4k.Q4K_ERR_ALIGN
    assert g(A, MIS, A, 16, 2048, 0, None) == q4k.Q4K_ERR_ALIGN
    assert g(A, A, MIS, 16, 2048, 0, None) == q4k.Q4K_ERR_ALIGN
    for o in (dict(unit_bytes=32), dict(waves_per_block=2), dict(column_groups=9),
              dict(column_groups=-1), dict(tiles_per_block=-2), dict(batch_bytes=64),
              dict(unit_bytes=64, batch_bytes=128)):
        cfg = q4k.q6k_launch(**o)
        assert lib.q6k_gemv_ex(A, A, A, 16, 2048, 0, ctypes.byref(cfg), None) == \
            q4k.Q4K_ERR_UNSUPPORTED, o
    # whole-line units need w aligned to 128 bytes; 256-byte batches need rows
    # without a phase (a stride that is a multiple of 128, with lines)
    cfg = q4k.q6k_launch(unit_bytes=128)
    assert lib.q6k_gemv_ex(A + 16, A, A, 16, 4096, 3456, ctypes.byref(cfg), None) == \
        q4k.Q4K_ERR_UNSUPPORTED
    cfg = q4k.q6k_launch(batch_bytes=256)
    assert lib.q6k_gemv_ex(A, A, A, 16, 4096, 0, ctypes.byref(cfg), None) == \
        q4k.Q4K_ERR_UNSUPPORTED
    d = lib.q6k_dequantize
    assert d(None, A, 16, 2048, 0, None) == q4k.Q4K_ERR_NULL
    assert d(A, A, 16, 300, 0, None) == q4k.Q4K_ERR_SHAPE
    assert d(A, MIS, 16, 2048, 0, None) == q4k.Q4K_ERR_ALIGN
    assert d(A, A, 16, 2048, 1000, None) == q4k.Q4K_ERR_SHAPE
    buf = np.zeros(4 * 1680, np.uint8)
    assert lib.q6k_load(A, buf.ctypes.data, buf.nbytes - 1, 4, 2048, 0, None) == q4k.Q4K_ERR_SIZE
    assert lib.q6k_load(None, buf.ctypes.data, buf.nbytes, 4, 2048, 0, None) == q4k.Q4K_ERR_NULL
    assert lib.q6k_load(A, buf.ctypes.data, buf.nbytes, 4, 2048, 1688, None) == q4k.Q4K_ERR_ALIGN
    assert lib.q6k_load(A, buf.ctypes.data, buf.nbytes, 4, 2048, 1664, None) == q4k.Q4K_ERR_SHAPE


@pytest.mark.parametrize("n,k,stride,aligned,unit,batch,groups,rpb,grid", [
    (32000, 4096, 0, True, 128, 128, 1, 128, 250),     # dense LM head: 3360-byte rows, lines
    (32000, 4096, 3456, True, 128, 256, 1, 128, 250),  # rows padded to whole lines
    (32000, 4096, 3456, False, 64, 256, 1, 128, 250),  # w not 128-byte aligned: 64-byte pieces
    (4096, 14336, 0, True, 128, 128, 8, 16, 256),      # FFN down: one tile a workgroup, 8 groups
    (256, 1024, 848, True, 128, 128, 4, 16, 16),       # four superblocks: four groups at most
    (128256, 4096, 0, True, 128, 128, 1, 512, 251),    # four tiles a wave
    (17, 2048, 0, False, 64, 256, 8, 16, 2),
])
def test_q6k_plan_automatic(n, k, stride, aligned, unit, batch, groups, rpb, grid):
    p = q4k.q6k_plan(n, k, stride, aligned, lds_max=163840)
    assert (p.unit_bytes, p.batch_bytes, p.column_groups, p.rows_per_block, p.grid,
            p.waves_per_block) == (unit, batch, groups, rpb, grid, 8)
    # x (1264 bytes a column) + eight rings of 16 x 560 bytes + the group sums
    assert p.lds_bytes == (k // 256) * 1264 + 8 * 16 * 560 + (rpb * groups * 8 if groups > 1 else 0)


def test_q6k_plan_lds_limit():
    assert q4k.q6k_plan(64, 18432, 0, True, lds_max=163840).lds_bytes <= 163840
    with pytest.raises(q4k.Q4KError) as e:
        q4k.q6k_plan(64, 18432 + 2048, 0, True, lds_max=163840)
    assert e.value.rc == q4k.Q4K_ERR_UNSUPPORTED
    p = q4k.q6k_plan(64, 16384, 0, True, lds_max=163840, waves_per_block=4)
    assert p.waves_per_block == 4 and p.lds_bytes == 64 * 1264 + 4 * 16 * 560 + (
        p.rows_per_block * p.column_groups * 8 if p.column_groups > 1 else 0)
    with pytest.raises(q4k.Q4KError):
        q4k.q6k_plan(64, 18432, 0, True, lds_max=163840, waves_per_block=4)   # x per thread


# ------------------------------------------------ fp16 mirror and prefill
def test_f16_refusals(lib):
    """Argument checks of the mirror, convert and GEMM entry points, before
    any HIP call."""
    assert lib.q4k_mirror_f16(None, A, 16, 256, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_mirror_f16(A, A, 16, 300, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_mirror_f16(A, MIS, 16, 256, None) == q4k.Q4K_ERR_ALIGN
    assert lib.q6k_mirror_f16(A, None, 16, 2048, 0, None) == q4k.Q4K_ERR_NULL
    assert lib.q6k_mirror_f16(A, A, 16, 2048, 1000, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q6k_mirror_f16(A, A, 16, 1024, 0, None) == q4k.Q4K_ERR_ALIGN   # 840-byte rows
    assert lib.q4k_f16_cvt(None, A, 16, None) == q4k.Q4K_ERR_NULL
    assert lib.q4k_f16_cvt(A, A, 0, None) == q4k.Q4K_ERR_SHAPE
    assert lib.q4k_f16_cvt(A, MIS, 16, None) == q4k.Q4K_ERR_ALIGN
    g = lib.q4k_f16_gemm
    assert g(None, A, A, 8, 8, 64, None) == q4k.Q4K_ERR_NULL
    assert g(A, A, None, 8, 8, 64, None) == q4k.Q4K_ERR_NULL
    for m, n, k in ((0, 8, 64), (8, 0, 64), (8, 8, 0), (2 ** 31, 8, 64)):
        assert g(A, A, A, m, n, k, None) == q4k.Q4K_ERR_SHAPE, (m, n, k)
    assert g(A, A, A, 8, 8, 96, None) == q4k.Q4K_ERR_UNSUPPORTED      # k % 64
    assert g(MIS, A, A, 8, 8, 64, None) == q4k.Q4K_ERR_ALIGN
    assert g(A, A, MIS, 8, 8, 64, None) == q4k.Q4K_ERR_ALIGN
    f = lib.q4k_f16_gemm_f32x
    assert f(A, None, A, A, 8, 8, 64, None) == q4k.Q4K_ERR_NULL
    assert f(A, A, None, A, 8, 8, 64, None) == q4k.Q4K_ERR_NULL
    assert f(A, MIS, A, A, 8, 8, 64, None) == q4k.Q4K_ERR_ALIGN
    assert f(A, A, A, A, 8, 8, 100, None) == q4k.Q4K_ERR_UNSUPPORTED

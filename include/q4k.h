/*
 * q4k.h -- C ABI of libq4k.so: the Q4_K fused dequantize-and-multiply GEMV
 * y = W.x for AMD Instinct MI355X (gfx950).
 *
 * The problem, as the pages state it:
 *  - W is n x k, stored as GGUF Q4_K: each row is k/256 superblocks of 144
 *    bytes (memra-engine 0.83.1, src/f16_ffi.rs: doc comment of
 *    `memra_q4_K_dequant_f16`, row-size check in `ensure_f16_mirror`); k must
 *    be a multiple of 256 (realizar 0.8.5, q4k_gemv_cached.rs: argument list
 *    of `q4k_gemv_cached`; uses.rs: `batched_q4k_gemv_into`).
 *  - Superblock layout (problem statement; not printed on the pages): bytes
 *    0-1 fp16 d, 2-3 fp16 dmin (little-endian), 4-15 the packed 6-bit
 *    (sc_j, m_j) pairs of the eight 32-element sub-blocks (GGUF K-quant
 *    packing), 16-143 the 4-bit codes: byte 32c+i holds element 64c+i in its
 *    low nibble and element 64c+32+i in its high nibble.  Each weight is
 *    w = d*sc_j*q - dmin*m_j.
 *  - x is m x k and y is m x n, both f32 row-major ("token-major"): vector b
 *    occupies x[b*k .. b*k+k-1] and y[b*n .. b*n+n-1] (realizar 0.8.5,
 *    uses.rs: memory-layout doc of `batched_q4k_gemv_into`; turbospark-
 *    runtime 0.1.0, real_forward_dispatch.rs: doc of `encode_gemm_any`).
 *    The pages batch at most 8 vectors per call (uses.rs:
 *    `batched_q4k_gemv_into`, "max 8"), except for 16 and 32, which share
 *    one weight stream between warps (uses.rs: `batched_q4k_gemv_into` and
 *    `batched_q4k_gemv_into_multi_warp`); here any 9-32 run, in one pass
 *    over the weights, where the kernels that can hold them apply.
 *    Anything else is refused by name, never looped (real_forward_dispatch.rs:
 *    doc of `encode_gemm_any`).
 *  - Weights are uploaded once and reused by every call (realizar 0.8.5,
 *    q4k_gemv_cached.rs: doc of `q4k_gemv_cached`); the launch is
 *    asynchronous on the caller's stream and the caller synchronises
 *    (q4k_gemv_cached.rs: `q4k_gemv_launch_to_ptr`); the output is a
 *    caller-owned, pre-allocated buffer that is fully overwritten (uses.rs:
 *    doc of `q4k_gemv_into_tiled`).
 *  - Pointers are validated before anything is launched (q4k_gemv_cached.rs:
 *    `q4k_gemv_indexed_async`; uses.rs: `validate_device_ptr` calls), and
 *    errors come back as an integer status across the C ABI (memra-engine
 *    0.83.1, src/f16_ffi.rs: the `extern "C"` block and the status decode in
 *    `qmatvec_gemm_f16_raw`).
 *
 * Conventions for every entry point:
 *  - Device pointers are plain HIP device addresses (e.g. from a torch
 *    tensor's data_ptr()); host pointers are ordinary process memory.  The
 *    library never takes ownership and never frees anything.
 *  - `stream` is a hipStream_t (NULL = the default stream).
 *  - Return value: Q4K_OK (0) or one of the codes below.  Argument errors are
 *    detected before any HIP call and nothing is launched; nothing aborts or
 *    throws across the ABI.  A failing HIP call returns Q4K_ERR_HIP plus the
 *    hipError_t value.
 *  - Calls are thread-safe.  The library's only state is set once per
 *    device and read atomically: the device's LDS limit and the address of
 *    the scratch array of q4k_f16_gemm_f32x_noalloc (whose calls, unlike
 *    every other entry point's, share that array; see there).
 */
#ifndef Q4K_H
#define Q4K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum q4k_status {
    Q4K_OK = 0,
    Q4K_ERR_NULL = 1,        /* a required pointer is NULL                       */
    Q4K_ERR_SHAPE = 2,       /* n < 1, k < 256, k % 256 != 0, m < 1, or too big  */
    Q4K_ERR_SIZE = 3,        /* byte count does not match n rows of the format   */
    Q4K_ERR_ALIGN = 4,       /* a pointer (or a Q6_K row stride) is not 16-byte
                                aligned                                         */
    Q4K_ERR_UNSUPPORTED = 5, /* m > 32; 9-32 vectors where the one-pass
                                kernels 5-7 do not apply; or a launch
                                option that cannot be honoured                  */
    Q4K_ERR_HIP = 1000       /* + hipError_t                                     */
};

/* Bytes of one Q4_K row of k weights: (k/256)*144, or 0 when k < 256 or
 * k % 256 != 0 (memra-engine 0.83.1, src/f16_ffi.rs, `ensure_f16_mirror`:
 * row_bytes == (in_f/256)*144). */
size_t q4k_row_bytes(int64_t k);

/* Copy n rows of GGUF Q4_K bytes, unchanged, from host memory `src_host`
 * (`src_bytes` long) into the caller's device buffer `w_dev`, which must hold
 * at least n*q4k_row_bytes(k) bytes and be 16-byte aligned.  Synchronous on
 * `stream`: the host buffer may be freed on return.  Errors: NULL pointers,
 * bad shape, src_bytes != n*q4k_row_bytes(k) (overflow-checked), alignment. */
int q4k_load(void* w_dev, const void* src_host, size_t src_bytes,
             int64_t n, int64_t k, void* stream);

/* y[b*n + r] = sum_c W[r][c] * x[b*k + c]  for b < m, r < n.
 *  w : device, n*(k/256)*144 bytes of Q4_K rows, 16-byte aligned
 *  x : device, m*k f32, 16-byte aligned
 *  y : device, m*n f32, 16-byte aligned, fully overwritten (no accumulate)
 *  1 <= n <= 2^31-1, 256 <= k <= 2^31-1 with k % 256 == 0, 1 <= m <= 8.
 *  9 <= m <= 32 (beyond the pages' batch of 8): one pass over the weights on
 *  the sub-block matrix-core kernels (5-7 up to 16 vectors, 6 beyond) when
 *  w is 128-byte aligned and their LDS fits; otherwise Q4K_ERR_UNSUPPORTED.
 *  m > 32: Q4K_ERR_UNSUPPORTED.  A batch is never split into several launches.
 * Asynchronous on `stream`; allocates nothing.  Results agree with the exact
 * dot product of the dequantized weights within 1e-5 * sum|w||x| per output
 * for every input whose exact result is finite (the tolerance the problem
 * states); where the exact result is an infinity or NaN, so is y.
 * Dequantization happens in registers; the weights are read exactly once
 * from HBM. */
int q4k_gemv(const void* w, const float* x, float* y,
             int64_t n, int64_t k, int64_t m, void* stream);

/* out[r*k + c] = W[r][c] as f32 (bit-exact: one round-to-nearest-even of
 * d*sc_j*q - dmin*m_j, whose products are exact in f32).  The f32 twin of the
 * pages' Q4_K dequantizer (memra-engine 0.83.1, src/f16_ffi.rs: doc comment
 * of `memra_q4_K_dequant_f16`, which writes the same weights as fp16 for a
 * mirror of the matrix).
 *  w   : device, as for q4k_gemv
 *  out : device, n*k f32, 16-byte aligned.
 * Asynchronous on `stream`. */
int q4k_dequantize(const void* w, float* out, int64_t n, int64_t k, void* stream);

/* The integer-dot variant: the Q8 quantize kernel and the DP4A Q4_K GEMV
 * that realizar 0.8.5 preloads together (src/cuda/executor/layers/
 * modules_utilities.rs, `preload_hw_dp4a_modules`), fused into one launch.
 * x is quantized inside the kernel in blocks of 32 consecutive elements
 * (one Q4_K sub-block; the block format is a reading, the pages name the
 * kernels only): d = amax/127 in f32, amax the largest |x| of the block (NaN
 * when the block holds a NaN), int8 codes q = nearest-even integer of
 * x * (127/amax) (quotient and product rounded to f32; 0 where amax is 0
 * or NaN, or the product is not finite) -- exactly what q4k_quantize_q8
 * writes.  Then y = sum_c w * d * q with exact int32 code sums, each
 * sub-block rounded once in f64 at its scale d, and y rounded once to f32.
 *  w : device, as for q4k_gemv, 128-byte aligned (whole-line reads)
 *  x : device, k f32, 16-byte aligned;  y : device, n f32, 16-byte aligned,
 *  overwritten.  m must be 1 (Q4K_ERR_UNSUPPORTED otherwise); k as for
 *  q4k_gemv, at most 4096 * 4 * 8 (x staged whole).
 * Its own tolerance (not q4k_gemv's): |y - y_ref| <= sum_e |w_e| (d_b(e)/2 *
 * (1 + 2^-19) + 2^-20 |x_e|) + 2^-23 |y_ref|, y_ref the exact GEMV with the
 * f32 x (a code carries its x to within d/2 (1 + 2^-20) + 2^-21 |x|);
 * against the exact GEMV of the quantized x (d*q) it is within
 * 2^-23 |y| + 1e-9 sum|w||d q|.  Non-finite x make y NaN.  Asynchronous on
 * `stream`; allocates nothing. */
int q4k_gemv_q8(const void* w, const float* x, float* y, int64_t n, int64_t k, int64_t m,
                void* stream);

/* The Q8 quantization of q4k_gemv_q8 on its own (tests, and callers that
 * keep x in Q8): q[b*k + c] int8 codes and d[b*(k/32) + c/32] f32 scales of
 * the m vectors of x (m x k f32).  All three pointers device and 16-byte
 * aligned; k a positive multiple of 32.  Asynchronous on `stream`. */
int q4k_quantize_q8(const float* x, int8_t* q, float* d, int64_t k, int64_t m, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* q4k_status_string(int rc);

/* ---------------------------------------------------------------------
 * Launch options for q4k_gemv_ex (tests and tuning).  q4k_gemv is
 * q4k_gemv_ex with every field 0 (automatic).  Kernels:
 *   1  x-stager (any m): x staged in LDS (whole or in K-chunks), fp32 decode
 *   2  streaming (m = 1): rows streamed with dwordx4 loads, fp32 decode
 *   3  line-streamed vector-ALU (m = 1): whole 128-byte weight lines through
 *      a per-wave LDS ring, int8 dot products with x broadcast by DPP
 *   4  line-streamed int8 matrix-core (m <= 8), one MFMA group per vector
 *   5  sub-block int8 matrix-core (m <= 16), one MFMA per sub-block and quad
 *      of vectors
 *   6  kernel 5 with x converted one superblock column at a time by each
 *      wave for itself (no whole x stage: any k and m; the only kernel for
 *      17-32 vectors, eight quads on four waves)
 *   7  kernel 5 with x converted once per workgroup, one column ahead, into
 *      a two-column window of every slab (one slab per task, eight waves;
 *      limits below; 16 * (8 / slabs) rows per workgroup by default)
 * Kernels 3-7 need w 128-byte aligned and their staged x plus line rings
 * within the LDS; kernels 4 and 7 also k % 2048 == 0 (rows of whole
 * 8-superblock slabs); kernels 3, 5 and 6 take rows of partial slabs too
 * (four-line rings, three lines in flight), kernel 3 up to k = 4096 *
 * waves_per_block.  Kernel 7: k / 2048 slabs times the vector quads (one
 * per four vectors) at most 8, slabs times the tiles of 16 rows of a
 * workgroup at most 8.
 * Automatic choice: m = 1 kernel 3 when it applies and the weights take at
 * least 16 MiB, else kernel 2 (the matrix cores only when asked for); m > 1
 * kernel 5 for m >= 3, kernel 4 for m = 2, the other of the two if only it
 * fits, else kernel 7, else kernel 6 when it fits, else kernel 1 (m <= 8).
 * With kernel = 0 and
 * another field set, m = 1 uses the streaming kernel and m > 1 the
 * x-stager.
 *
 * x is staged in LDS in spans of 4096 elements per vector.  The single-stage
 * variant holds all of x at once; the K-chunked variant stages
 * `spans_per_chunk` spans at a time and keeps each lane's partial sums
 * between chunks, so both variants accumulate in the same order and give
 * bit-identical y (realizar 0.8.5, q4k_gemv_cached.rs: the tiled / chunked
 * selection in `q4k_gemv_cached`; the automatic rule stages all of x at once
 * when it fits 48 KiB, the pages' 12288-float shared-memory limit).
 * ------------------------------------------------------------------- */
typedef struct q4k_launch {
    int32_t variant;          /* 0 automatic, 1 single-stage, 2 K-chunked          */
    int32_t spans_per_chunk;  /* K-chunked: spans per stage, >= 1 (0 = automatic)  */
    int32_t rows_per_block;   /* rows per workgroup (0 = automatic)                */
    int32_t rows_per_wave;    /* rows a wave decodes per pass: 0 auto, 1, 2 or 4   */
    int32_t waves_per_block;  /* 0 auto, 4 or 8                                    */
    int32_t x_in_registers;   /* 0 auto, 1 keep x in VGPRs (one span, m = 1), 2 LDS */
    int32_t kernel;           /* 0 auto, else 1-7 as listed above                  */
    int32_t ring_depth;       /* loads in flight per wave, 0 auto: streaming 1..4
                                 rows; line-streamed 3 or 9 lines                  */
    int32_t rows_per_task;    /* streaming: rows per wave task, 0 auto, >= 1       */
    int32_t cols_per_task;    /* line-streamed: superblock columns per task (whole
                                 slabs of 8 dividing the row), 0 auto              */
} q4k_launch;

/* q4k_gemv with explicit launch options (NULL = automatic).  Options that do
 * not fit the shape (e.g. single-stage when x exceeds the LDS limit) return
 * Q4K_ERR_UNSUPPORTED without launching. */
int q4k_gemv_ex(const void* w, const float* x, float* y,
                int64_t n, int64_t k, int64_t m,
                const q4k_launch* opts, void* stream);

/* The launch q4k_gemv_ex(w, x, y, n, k, m, opts, stream) would make,
 * without launching (introspection for tests and tuning).
 *   w_aligned128 : nonzero if the weights' address is 128-byte aligned (the
 *                  line-streamed kernels 3-6 need it)
 *   lds_max      : LDS bytes a workgroup may use; 0 = ask the current HIP
 *                  device (163840 on MI355X), so with a nonzero value no
 *                  HIP call is made and this runs without a GPU
 *   out          : host, filled on Q4K_OK
 * Returns what q4k_gemv_ex would return for the shape and options before
 * launching (Q4K_ERR_SHAPE, Q4K_ERR_UNSUPPORTED, ...); pointers and their
 * 16-byte alignment are not checked here. */
typedef struct q4k_plan_info {
    int32_t kernel;          /* 1-7 as listed above                           */
    int32_t grid;            /* workgroups                                     */
    int32_t threads;         /* per workgroup                                  */
    int32_t lds_bytes;       /* dynamic LDS per workgroup                      */
    int32_t rows_per_block;  /* weight rows per workgroup                      */
    int32_t cols_per_task;   /* line-streamed: superblock columns per task;
                                else 0                                          */
    int32_t ring_depth;      /* streaming: rows in flight; line-streamed: lines */
    int32_t spans_per_chunk; /* kernels 1, 2: 4096-element spans per x stage;
                                else 0                                          */
} q4k_plan_info;

int q4k_plan(int64_t n, int64_t k, int64_t m, const q4k_launch* opts, int w_aligned128,
             size_t lds_max, q4k_plan_info* out);

/* ---------------------------------------------------------------------
 * Q6_K: the same GEMV over the other block format of the decode loop, one
 * vector (realizar 0.8.5, q4k_gemv_cached.rs: doc of
 * `q6k_gemv_cached_async`, the Q6_K GEMV used for an LM head stored as
 * Q6_K; memra-engine 0.83.1, src/f16_ffi.rs: doc of `memra_q6_K_dequant_f16`
 * and the row-size check in `ensure_f16_mirror`: 210-byte superblocks of
 * 256 weights, k / 256 of them per row).
 *  - Superblock layout (GGUF Q6_K; not printed on the pages): bytes 0-127
 *    ql, the low four bits of the codes; 128-191 qh, the high two bits;
 *    192-207 sixteen signed 8-bit scales, scale s for elements 16s..16s+15;
 *    208-209 fp16 d (little-endian).  Element e = 128h + 32t + l (h < 2,
 *    t < 4, l < 32) keeps its low bits in ql byte 64h + 32(t%2) + l (low
 *    nibble for t < 2, high nibble for t >= 2) and its high bits in bits
 *    2t, 2t+1 of qh byte 32h + l; its weight is w = d*sc*(q - 32), an exact
 *    product in f32.
 *  - Row r starts at byte r*row_stride of w; row_stride = 0 means the dense
 *    q6k_row_bytes(k).  row_stride must be a multiple of 16 and at least
 *    q6k_row_bytes(k) (Q4K_ERR_SHAPE below it, Q4K_ERR_ALIGN when it is not
 *    a multiple of 16: dense rows qualify when k % 2048 == 0), and w must
 *    hold n*row_stride bytes (the last row's padding included).  With w
 *    128-byte aligned the kernel reads whole 128-byte lines of each row
 *    (from the line holding its first byte), else 64-byte pieces.
 * ------------------------------------------------------------------- */

/* Bytes of one dense Q6_K row of k weights: (k/256)*210, or 0 when k < 256
 * or k % 256 != 0. */
size_t q6k_row_bytes(int64_t k);

/* Copy n dense rows of GGUF Q6_K bytes (src_bytes == n*q6k_row_bytes(k))
 * from host memory into the device buffer w_dev at row_stride (0 = dense),
 * leaving the padding bytes of each row untouched.  Synchronous on
 * `stream`.  Errors as q4k_load, and the row_stride rules above. */
int q6k_load(void* w_dev, const void* src_host, size_t src_bytes, int64_t n, int64_t k,
             int64_t row_stride, void* stream);

/* y[r] = sum_c W[r][c] * x[c] for r < n, W in Q6_K rows.
 *  w : device, 16-byte aligned, rows as above
 *  x : device, k f32, 16-byte aligned
 *  y : device, n f32, 16-byte aligned, fully overwritten
 *  1 <= n <= 2^31-1, 256 <= k with k % 256 == 0; x is staged whole in LDS
 *  beside eight waves' rings, so k <= 18432 on MI355X (160 KiB of LDS);
 *  beyond: Q4K_ERR_UNSUPPORTED.
 * Asynchronous on `stream`; allocates nothing.  Tolerance as q4k_gemv:
 * within 1e-5 * sum|w||x| of the exact dot product of the f32 weights for
 * every input whose exact result is finite; inf and NaN propagate. */
int q6k_gemv(const void* w, const float* x, float* y, int64_t n, int64_t k,
             int64_t row_stride, void* stream);

/* Launch options of q6k_gemv_ex (tests and tuning; every field 0 =
 * automatic). */
typedef struct q6k_launch {
    int32_t unit_bytes;       /* bytes of a row per load instruction: 64, or 128
                                 (whole lines; w 128-byte aligned)             */
    int32_t batch_bytes;      /* bytes of each row per batch: 128 (unit 128), or
                                 256 (unit 64, or row_stride % 128 == 0)        */
    int32_t waves_per_block;  /* 4 or 8 (4: k <= 16384)                        */
    int32_t column_groups;    /* tasks per 16-row tile, splitting its columns:
                                 1 .. min(16, k/256)                           */
    int32_t tiles_per_block;  /* 16-row tiles per workgroup, >= 1              */
} q6k_launch;

int q6k_gemv_ex(const void* w, const float* x, float* y, int64_t n, int64_t k,
                int64_t row_stride, const q6k_launch* opts, void* stream);

/* The launch q6k_gemv_ex would make, without launching: lds_max as for
 * q4k_plan (0 = ask the device), w_aligned128 as for q4k_plan. */
typedef struct q6k_plan_info {
    int32_t unit_bytes;
    int32_t batch_bytes;
    int32_t waves_per_block;
    int32_t column_groups;
    int32_t rows_per_block;
    int32_t grid;
    int32_t lds_bytes;
} q6k_plan_info;

int q6k_plan(int64_t n, int64_t k, int64_t row_stride, int w_aligned128, const q6k_launch* opts,
             size_t lds_max, q6k_plan_info* out);

/* out[r*k + c] = W[r][c] as f32, bit-exact (every Q6_K weight is exact in
 * f32): the f32 twin of `memra_q6_K_dequant_f16` (memra-engine 0.83.1,
 * src/f16_ffi.rs).  w as for q6k_gemv; out device, n*k f32, 16-byte
 * aligned.  Asynchronous on `stream`. */
int q6k_dequantize(const void* w, float* out, int64_t n, int64_t k, int64_t row_stride,
                   void* stream);

/* ---------------------------------------------------------------------
 * Prefill beside the decode path: a row-major fp16 mirror of the weights
 * and an fp16 GEMM on the matrix cores for batches of many vectors
 * (memra-engine 0.83.1, src/f16_ffi.rs: `memra_q4_K_dequant_f16` and
 * `memra_q6_K_dequant_f16` build the mirror at load time, `memra_f16_cvt`
 * converts the f32 activations, `memra_f16_pp_gemm` runs
 * y[m, n] = x[m, k] @ (fp16 W)^T with f32 accumulation).
 *  - A mirror element is the f32 weight (as q4k_dequantize / q6k_dequantize
 *    give it) rounded to binary16, nearest even (beyond 65504: infinity);
 *    activations are rounded the same way.  The mirror takes 2 bytes per
 *    weight.
 *  - The GEMM's products of two binary16 values are exact in f32; its sums
 *    are f32, so y is within k * 2^-23 * sum|w16||x16| of the exact dot
 *    product of the fp16 operands (the bound of an f32 sum of k terms in any
 *    order, with a factor of 2 to spare).  Against the f32 weights and
 *    activations the fp16 roundings add up to 2^-10 sum|w||x| more: this is
 *    the numeric class of the pages' fp16 prefill lane, not q4k_gemv's.
 * ------------------------------------------------------------------- */

/* The fp16 mirror of n dense Q4_K rows: w16[r*k + c] = binary16 of W[r][c].
 * w device (16-byte aligned), w16 device, n*k halves, 16-byte aligned.
 * Asynchronous on `stream`. */
int q4k_mirror_f16(const void* w, void* w16, int64_t n, int64_t k, void* stream);

/* The fp16 mirror of n Q6_K rows at row_stride (0 = dense; the rules of
 * q6k_gemv). */
int q6k_mirror_f16(const void* w, void* w16, int64_t n, int64_t k, int64_t row_stride,
                   void* stream);

/* x16[i] = binary16 of x[i] (nearest even) for i < count: f32 in, fp16 out,
 * both device and 16-byte aligned.  Asynchronous. */
int q4k_f16_cvt(const float* x, void* x16, int64_t count, void* stream);

/* y[b*n + r] = sum_c w16[r*k + c] * x16[b*k + c] for b < m, r < n: the fp16
 * mirror w16 (n x k), fp16 activations x16 (m x k), y f32 (m x n, fully
 * overwritten).  All device, 16-byte aligned; m, n >= 1; k >= 64 with
 * k % 64 == 0 (Q4K_ERR_UNSUPPORTED otherwise).  Matrix cores
 * (v_mfma_f32_16x16x32_f16), f32 accumulation; asynchronous; allocates
 * nothing. */
int q4k_f16_gemm(const void* w16, const void* x16, float* y, int64_t m, int64_t n, int64_t k,
                 void* stream);

/* q4k_f16_cvt of the f32 activations x (m x k) into the caller's scratch xh
 * (m*k halves, 16-byte aligned), then q4k_f16_gemm: the pages' one-call
 * prefill GEMM (`memra_f16_pp_gemm`).  Asynchronous; allocates nothing. */
int q4k_f16_gemm_f32x(const void* w16, const float* x, void* xh, float* y, int64_t m,
                      int64_t n, int64_t k, void* stream);

/* q4k_f16_gemm_f32x without the scratch argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the fp16 activations go to a static device array
 * of the library, 4 Mi halves (8 MiB) on each device it runs on, held until
 * the process ends.  m*k above 4 * 2^20 returns Q4K_ERR_UNSUPPORTED before
 * any HIP call.  Nothing is allocated; the first call on a device looks the
 * array's address up (hipGetSymbolAddress).  Calls on one device share the
 * array: calls that overlap on one GPU (other streams, other threads) race
 * and must be serialised by the caller.  Asynchronous on `stream`. */
int q4k_f16_gemm_f32x_noalloc(const void* w16, const float* x, float* y, int64_t m, int64_t n,
                              int64_t k, void* stream);

/* Read `bytes` (a multiple of 16) of device memory at `buf` (16-byte
 * aligned) with coalesced 16-byte loads and write a checksum per workgroup
 * to `out` (device, q4k_read_calibrate_blocks() floats).  Benchmark
 * calibration: the achievable streaming-read rate.  Asynchronous. */
int q4k_read_calibrate(const void* buf, size_t bytes, float* out, void* stream);
int q4k_read_calibrate_blocks(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4K_H */

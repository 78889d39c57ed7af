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
 *    At most 8 vectors per call (uses.rs: `batched_q4k_gemv_into`, "max 8");
 *    more are refused by name, never looped (real_forward_dispatch.rs: doc of
 *    `encode_gemm_any`).
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
 *  - Calls are thread-safe: the library keeps no mutable state.
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
    Q4K_ERR_SIZE = 3,        /* byte count does not match n*(k/256)*144          */
    Q4K_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                 */
    Q4K_ERR_UNSUPPORTED = 5, /* m > 16, or a launch option that cannot be
                                honoured (m > 8: kernels 5 and 6 only)          */
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
 *  9 <= m <= 16: one pass over the weights for all m vectors on the
 *  sub-block matrix-core kernels (5, 6) where their whole x stage fits or
 *  eight vectors would need kernel 6 as well; otherwise two launches on
 *  `stream`, vectors 0-7 and then the rest (so any alignment and k).
 *  m > 16: Q4K_ERR_UNSUPPORTED.
 * Asynchronous on `stream`; allocates nothing.  Results agree with the exact
 * dot product of the dequantized weights within 1e-5 * sum|w||x| per output
 * on the workloads' value distributions.  Dequantization happens in
 * registers; the weights are read exactly once from HBM. */
int q4k_gemv(const void* w, const float* x, float* y,
             int64_t n, int64_t k, int64_t m, void* stream);

/* out[r*k + c] = W[r][c] as f32 (bit-exact: one round-to-nearest-even of
 * d*sc_j*q - dmin*m_j, whose products are exact in f32).
 *  w   : device, as for q4k_gemv
 *  out : device, n*k f32, 16-byte aligned.
 * Asynchronous on `stream`. */
int q4k_dequantize(const void* w, float* out, int64_t n, int64_t k, void* stream);

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
 *      wave for itself (no whole x stage: any k and m)
 * Kernels 3-6 need w 128-byte aligned and their staged x plus line rings
 * within the LDS; kernel 4 also k % 2048 == 0 (rows of whole 8-superblock
 * slabs); kernels 3, 5 and 6 take rows of partial slabs too (four-line
 * rings, three lines in flight), kernel 3 up to k = 4096 * waves_per_block.
 * Automatic choice: m = 1 kernel 3 when it applies and the weights take at
 * least 16 MiB, else kernel 2 (the matrix cores only when asked for); m > 1
 * kernel 5 for m >= 3, kernel 4 for m = 2, the other of the two if only it
 * fits, else kernel 6 when it fits, else kernel 1 (m <= 8).  With kernel = 0 and
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
    int32_t waves_per_block;  /* 0 auto, 4 or 8; 16 for kernels 2-4 at m = 1       */
    int32_t x_in_registers;   /* 0 auto, 1 keep x in VGPRs (one span, m = 1), 2 LDS */
    int32_t kernel;           /* 0 auto, else 1-6 as listed above                  */
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
    int32_t kernel;          /* 1-6 as listed above                           */
    int32_t grid;            /* workgroups                                     */
    int32_t threads;         /* per workgroup                                  */
    int32_t lds_bytes;       /* dynamic LDS per workgroup                      */
    int32_t rows_per_block;  /* weight rows per workgroup                      */
    int32_t cols_per_task;   /* line-streamed: superblock columns per task;
                                else 0                                          */
    int32_t ring_depth;      /* streaming: rows in flight; line-streamed: lines */
    int32_t spans_per_chunk; /* kernels 1, 2: 4096-element spans per x stage;
                                else 0                                          */
    int32_t launches;        /* 1; 2 when an automatic plan of 9-16 vectors
                                launches vectors 0-7, then the rest (the fields
                                above describe the first launch)               */
} q4k_plan_info;

int q4k_plan(int64_t n, int64_t k, int64_t m, const q4k_launch* opts, int w_aligned128,
             size_t lds_max, q4k_plan_info* out);

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

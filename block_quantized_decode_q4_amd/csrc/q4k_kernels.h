// q4k_kernels.h -- internal interface between the C-ABI layer (q4k_api.hip)
// and the kernels (q4k_kernels.hip, q4k_dpp.hip, q4k_mfma.hip, q4k_q8.hip,
// q4k_q6k.hip, q4k_f16.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q4k {

constexpr int kQK = 256;          // weights per superblock
constexpr int kBlockBytes = 144;  // bytes per superblock
constexpr int kSpanSB = 16;       // superblocks per wave pass (4 lanes each)
constexpr int kSpan = kSpanSB * kQK;
constexpr int kMaxM = 8;         // vectors per launch that every kernel takes
constexpr int kMaxMStaged = 16;  // kernels 5 and 7: x of at most four vector quads in LDS
constexpr int kMaxMWide = 32;    // kernel 6 (eight quads, x per wave and column)
constexpr int kReadBlocks = 1024;    // four 512-lane workgroups per CU of a 256-CU part
constexpr int kReadThreads = 512;

// One resolved launch of the GEMV kernel.
struct GemvPlan {
    int n, k, S, m;
    int nspans;            // ceil(S / 16)
    int spans_per_chunk;   // spans of x staged at once (== nspans: single-stage)
    int nchunks;
    int rows_per_block;
    int rows_per_wave;     // R: 1, 2 or 4 (4 only for m = 1)
    int waves_per_block;   // 4 or 8
    int x_in_registers;    // 1: x kept in VGPRs (single span, m = 1)
    int grid;
    size_t lds_bytes;
    int kernel;            // 1: x-stager, 2: streaming, 3: line-streamed int8 dot products
                           // (vector ALU), 4: line-streamed int8 matrix-core,
                           // 5: sub-block int8 matrix-core, 6: the same with x
                           // converted per column by each wave
    int ring_depth;        // kernel 2: rows in flight per wave; 3-6: lines in flight
    int rows_per_task;     // streaming kernel: rows per wave task
    int cols_per_task;     // line-streamed kernels: superblock columns per task
};

hipError_t launch_gemv(const GemvPlan& p, const void* w, const float* x, float* y,
                       hipStream_t stream);
hipError_t launch_gemv_mfma(const GemvPlan& p, const void* w, const float* x, float* y,
                            hipStream_t stream);
size_t lines_lds_bytes(int S, int m, int waves);
size_t sub_lds_bytes(int S, int m);
size_t jit_lds_bytes(int S, int m);
int jit_waves(int m);      // waves per workgroup of kernel 6 for m vectors
size_t win_lds_bytes(int S, int m);
hipError_t launch_gemv_dot4(const GemvPlan& p, const void* w, const float* x, float* y,
                            hipStream_t stream);
size_t dot4_lds_bytes(int S, int waves);
hipError_t launch_dequant(const void* w, float* out, int64_t nsb, hipStream_t stream);
// the integer-dot variant with x quantized to Q8 (q4k_q8.hip)
hipError_t launch_gemv_q8(const GemvPlan& p, const void* w, const float* x, float* y,
                          hipStream_t stream);
hipError_t launch_quantize_q8(const float* x, int8_t* q, float* d, int64_t nblocks,
                              hipStream_t stream);
size_t q8_lds_bytes(int S, int waves);
hipError_t launch_read(const void* buf, size_t n16, float* out, hipStream_t stream);

// The GEMV over Q6_K weights (q4k_q6k.hip), one vector.
struct Q6kPlan {
    int n, k, S;
    int64_t row_stride;    // bytes from one row to the next (a multiple of 16)
    int unit;              // bytes of a row one load instruction reads: 64, or 128
                           // (whole lines; w 128-byte aligned)
    int batch;             // bytes of a row per batch: 256 (no row has a phase within
                           // its line: unit 64, or a row stride that is a multiple
                           // of 128) or 128
    int waves_per_block;   // 8, or 4 when the LDS cannot hold eight rings
    int rows_per_block;    // 16 per tile
    int ncg;               // column groups per tile (the tasks of one tile)
    int grid;
    size_t lds_bytes;
};
hipError_t launch_q6k_gemv(const Q6kPlan& p, const void* w, const float* x, float* y,
                           hipStream_t stream);
hipError_t launch_q6k_dequant(const void* w, float* out, int64_t n, int S, int64_t row_stride,
                              hipStream_t stream);
size_t q6k_lds_bytes(int S, int waves, int rows_per_block, int ncg);

// The fp16 mirror and the prefill GEMM (q4k_f16.hip; mirror builds in
// q4k_kernels.hip and q4k_q6k.hip).
hipError_t launch_dequant_f16(const void* w, void* out, int64_t nsb, hipStream_t stream);
hipError_t launch_q6k_dequant_f16(const void* w, void* out, int64_t n, int S, int64_t row_stride,
                                  hipStream_t stream);
hipError_t launch_f16_cvt(const float* x, void* out, int64_t count, hipStream_t stream);
hipError_t launch_f16_gemm(const void* w16, const void* x16, float* y, int m, int n, int k,
                           hipStream_t stream);
void f16_gemm_tile(int64_t m, int64_t n, int* bm, int* bn);
// the static scratch of q4k_f16_gemm_f32x_noalloc: 4 Mi halves (8 MiB) per
// device; f16_scratch gives its device address on the current device
constexpr int64_t kScratchHalves = (int64_t)4 << 20;
hipError_t f16_scratch(void** out);
size_t f16_gemm_lds_bytes(int bm, int bn);
int64_t f16_gemm_grid(int64_t m, int64_t n);

}  // namespace q4k

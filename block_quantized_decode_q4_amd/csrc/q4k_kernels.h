// q4k_kernels.h -- internal interface between the C-ABI layer (q4k_api.hip)
// and the kernels (q4k_kernels.hip, q4k_dpp.hip, q4k_mfma.hip).  Not
// installed, not part of the ABI.
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
constexpr int kMaxMWide = 16;    // the sub-block matrix-core kernels 5 and 6
constexpr int kReadBlocks = 4096;

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
hipError_t launch_gemv_dot4(const GemvPlan& p, const void* w, const float* x, float* y,
                            hipStream_t stream);
size_t dot4_lds_bytes(int S, int waves);
hipError_t launch_dequant(const void* w, float* out, int64_t nsb, hipStream_t stream);
hipError_t launch_read(const void* buf, size_t n16, float* out, hipStream_t stream);

}  // namespace q4k

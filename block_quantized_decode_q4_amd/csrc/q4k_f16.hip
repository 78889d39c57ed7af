// q4k_f16.hip -- the prefill step beside the decode GEMV: a row-major fp16
// mirror of the weights (built by the dequant kernels of q4k_kernels.hip and
// q4k_q6k.hip) times fp16 activations on the matrix cores, f32 accumulation
// (memra-engine 0.83.1, src/f16_ffi.rs: `memra_f16_cvt`, the f32 -> fp16
// activation convert; `memra_f16_pp_gemm` / `try_f16_gemm`,
// y[m, n] = x[m, k] @ (fp16 W)^T, f32 accumulate, for prefill batches).
//
// GEMM: a 256-thread workgroup computes a 128 x 128 tile of y (128 vectors x
// 128 weight rows; 64 x 128 or 64 x 64 when that gives too few tiles to
// fill the chip) over k in steps of 64: both operands are k-contiguous
// (x rows and mirror rows), staged through LDS in rows of 64 halves padded
// to 144 bytes (consecutive rows start 16 bytes apart in the banks), two
// LDS stages and two register sets of loaded tiles, so a step's global
// loads have two steps of MFMAs to arrive in.  (Mirror blocks loaded by
// each wave straight into its operand registers, with only x staged,
// measured 1.5-2.3 x slower.)  Wave
// (wm, wn) of the 2 x 2 layout holds a quarter of the tile (64 x 64 for
// 128 x 128) as 16 x 16 blocks of v_mfma_f32_16x16x32_f16 accumulators: lane l = 16 g + j holds
// A[i = j][k = 8 g .. 8 g + 7] (an x row), B[k = 8 g .. 8 g + 7][j] (a
// mirror row) and D[4 g + r][j].  Workgroups that share a block of mirror
// rows run on the same XCD one after another (its L2 serves the repeats):
// the mirror, the large operand, is read from HBM about once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>
#include <mutex>

#include "q4k_kernels.h"

namespace q4k {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

constexpr int kGK = 64;                  // k per step
constexpr int kGRow = kGK * 2 + 16;      // LDS bytes per staged row (padded)
constexpr int kGXcd = 8;                 // XCDs: workgroups go round-robin over them

// f32 -> fp16, round to nearest even (inf beyond the fp16 range, NaN kept).
__global__ void __launch_bounds__(256)
f16_cvt_kernel(const float* __restrict__ x, _Float16* __restrict__ out, int64_t count)
{
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i + 4 <= count) {
        const float4 v = *reinterpret_cast<const float4*>(x + i);
        typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
        const h4_t h = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
        *reinterpret_cast<h4_t*>(out + i) = h;
    } else {
        for (int64_t t = i; t < count; ++t) {
            out[t] = (_Float16)x[t];
        }
    }
}

// y[b * n + r] = sum_c w16[r * k + c] x16[b * k + c] (f32 accumulation).
// Tiles of BM x rows by BN mirror rows (64 or 128 each); four waves in a
// 2 x 2 layout, each with (BM / 32) x (BN / 32) MFMA blocks of 16 x 16.
// Grid: kGXcd * ceil(NT / kGXcd) * MT workgroups (MT, NT: tiles of x rows
// and of mirror rows); k % 64 == 0.
template <int BM, int BN>
__global__ void __launch_bounds__(256, 2)
f16_gemm_kernel(const _Float16* __restrict__ w16, const _Float16* __restrict__ x16,
                float* __restrict__ y, int m, int n, int k, int MT, int NT)
{
    static_assert((BM == 64 || BM == 128) && (BN == 64 || BN == 128), "tile");
    constexpr int LA = BM / 32;              // 16-byte loads of the x tile per thread and step
    constexpr int LB = BN / 32;
    constexpr int FA = BM / 32;              // 16-row MFMA blocks per wave
    constexpr int FB = BN / 32;
    constexpr int kXs = BM * kGRow;          // LDS bytes of one x tile
    constexpr int kStage = (BM + BN) * kGRow;
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // XCD-aware tile order: workgroup b runs on XCD b % 8; within an XCD
    // the x tiles of one mirror tile follow each other
    const int bid = blockIdx.x;
    const int xcd = bid % kGXcd;
    const int local = bid / kGXcd;
    const int tm = local % MT;
    const int tn = (local / MT) * kGXcd + xcd;
    if (tn >= NT) {
        return;
    }
    const int row_x0 = tm * BM;
    const int row_w0 = tn * BN;

    // load role: 16 bytes of a tile row per thread and load (tile row
    // idx / 8, 16-byte chunk idx % 8 of its 128 bytes)
    const _Float16* xsrc[LA];
    const _Float16* wsrc[LB];
    int xoff[LA], woff[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int idx = tid + 256 * i;
        xsrc[i] = x16 + (int64_t)min(row_x0 + (idx >> 3), m - 1) * k + (idx & 7) * 8;
        xoff[i] = (idx >> 3) * kGRow + (idx & 7) * 16;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int idx = tid + 256 * i;
        wsrc[i] = w16 + (int64_t)min(row_w0 + (idx >> 3), n - 1) * k + (idx & 7) * 8;
        woff[i] = kXs + (idx >> 3) * kGRow + (idx & 7) * 16;
    }
    // kSets register sets of loaded tiles: a set is refilled with the loads
    // of step kb + 1 + kSets right after its tiles of step kb + 1 are staged,
    // so a load has kSets steps of MFMAs to arrive in
    constexpr int kSets = 2;
    static_assert(kSets == 2, "the step loop below alternates two sets");
    v4u_t xa[kSets][LA], wa[kSets][LB];
    auto load = [&](int kb, auto set) __attribute__((always_inline)) {
        constexpr int q = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            xa[q][i] = *reinterpret_cast<const v4u_t*>(xsrc[i] + kb * kGK);
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            wa[q][i] = *reinterpret_cast<const v4u_t*>(wsrc[i] + kb * kGK);
        }
    };
    auto stage = [&](int st, auto set) __attribute__((always_inline)) {
        constexpr int q = decltype(set)::value;
        unsigned char* base = smem + st * kStage;
#pragma unroll
        for (int i = 0; i < LA; ++i) {
            *reinterpret_cast<v4u_t*>(base + xoff[i]) = xa[q][i];
        }
#pragma unroll
        for (int i = 0; i < LB; ++i) {
            *reinterpret_cast<v4u_t*>(base + woff[i]) = wa[q][i];
        }
    };

    // compute role: wave (wm, wn), lane (g, j)
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int g = lane >> 4;
    const int j = lane & 15;
    f32x4_t acc[FA][FB];
#pragma unroll
    for (int a = 0; a < FA; ++a) {
#pragma unroll
        for (int b = 0; b < FB; ++b) {
            acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
    const int KB = k / kGK;
    // set q holds steps q, q + kSets, q + 2 kSets, ...  Prologue: steps
    // 0 .. kSets - 1 into the sets (past the end the last step again: no
    // branch around a load), step 0 staged and its set refilled with step
    // kSets
    load(0, std::integral_constant<int, 0>());
    load(min(1, KB - 1), std::integral_constant<int, 1>());
    stage(0, std::integral_constant<int, 0>());
    load(min(kSets, KB - 1), std::integral_constant<int, 0>());
    __syncthreads();
    // step kb: its tiles are in LDS stage kb & 1; set (kb + 1) % kSets holds
    // step kb + 1, staged after the MFMAs into the other stage and then
    // refilled with step kb + 1 + kSets
    auto step = [&](int kb, auto nset) __attribute__((always_inline)) {
        const int st = kb & 1;
        const unsigned char* xs = smem + st * kStage;
        const unsigned char* ws = xs + kXs;
#pragma unroll
        for (int s = 0; s < kGK / 32; ++s) {
            half8_t av[FA], bv[FB];
#pragma unroll
            for (int a = 0; a < FA; ++a) {
                av[a] = *reinterpret_cast<const half8_t*>(
                    xs + ((BM / 2) * wm + 16 * a + j) * kGRow + (32 * s + 8 * g) * 2);
            }
#pragma unroll
            for (int b = 0; b < FB; ++b) {
                bv[b] = *reinterpret_cast<const half8_t*>(
                    ws + ((BN / 2) * wn + 16 * b + j) * kGRow + (32 * s + 8 * g) * 2);
            }
#pragma unroll
            for (int a = 0; a < FA; ++a) {
#pragma unroll
                for (int b = 0; b < FB; ++b) {
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[a], bv[b], acc[a][b],
                                                                       0, 0, 0);
                }
            }
        }
        stage(st ^ 1, nset);
        load(min(kb + 1 + kSets, KB - 1), nset);
        __syncthreads();
    };
    for (int kb = 0; kb < KB; kb += kSets) {
        step(kb, std::integral_constant<int, 1>());
        if (kb + 1 < KB) {
            step(kb + 1, std::integral_constant<int, 0>());
        }
    }
    // D[4 g + r][j] of block (a, b): x row (BM / 2) wm + 16 a + 4 g + r,
    // mirror row (BN / 2) wn + 16 b + j
#pragma unroll
    for (int a = 0; a < FA; ++a) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int xr = row_x0 + (BM / 2) * wm + 16 * a + 4 * g + r;
            if (xr < m) {
#pragma unroll
                for (int b = 0; b < FB; ++b) {
                    const int wr = row_w0 + (BN / 2) * wn + 16 * b + j;
                    if (wr < n) {
                        y[(int64_t)xr * n + wr] = acc[a][b][r];
                    }
                }
            }
        }
    }
}

hipError_t launch_f16_cvt(const float* x, void* out, int64_t count, hipStream_t stream)
{
    const int64_t blocks = (count + 1023) / 1024;
    hipLaunchKernelGGL(f16_cvt_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       static_cast<_Float16*>(out), count);
    return hipGetLastError();
}

// The tile: 128 x 128 while that gives at least 384 tiles (about 1.5 per
// CU), else 64 x 128 while that gives a tile for every CU (a wave's 32 x 64
// block reads a third less LDS per flop than 32 x 32: m 512, n 4096,
// k 14336 in 100 us against 105 us on 64 x 64), else 64 x 64 (more,
// smaller tiles for short m or n with long k).
void f16_gemm_tile(int64_t m, int64_t n, int* bm, int* bn)
{
    auto tiles = [&](int a, int b) { return ((m + a - 1) / a) * ((n + b - 1) / b); };
    if (tiles(128, 128) >= 384) {
        *bm = 128; *bn = 128;
    } else if (tiles(64, 128) >= 256) {
        *bm = 64; *bn = 128;
    } else {
        *bm = 64; *bn = 64;
    }
}

size_t f16_gemm_lds_bytes(int bm, int bn)
{
    return (size_t)2 * (bm + bn) * kGRow;
}

int64_t f16_gemm_grid(int64_t m, int64_t n)
{
    int bm, bn;
    f16_gemm_tile(m, n, &bm, &bn);
    const int64_t MT = (m + bm - 1) / bm;
    const int64_t NT = (n + bn - 1) / bn;
    return kGXcd * ((NT + kGXcd - 1) / kGXcd) * MT;
}

template <int BM, int BN>
static hipError_t launch_f16_gemm_t(const void* w16, const void* x16, float* y, int m, int n,
                                    int k, hipStream_t stream)
{
    const int MT = (m + BM - 1) / BM;
    const int NT = (n + BN - 1) / BN;
    const int64_t grid = kGXcd * ((int64_t)(NT + kGXcd - 1) / kGXcd) * MT;
    hipLaunchKernelGGL((f16_gemm_kernel<BM, BN>), dim3((unsigned)grid), dim3(256),
                       f16_gemm_lds_bytes(BM, BN), stream, static_cast<const _Float16*>(w16),
                       static_cast<const _Float16*>(x16), y, m, n, k, MT, NT);
    return hipGetLastError();
}

hipError_t launch_f16_gemm(const void* w16, const void* x16, float* y, int m, int n, int k,
                           hipStream_t stream)
{
    int bm, bn;
    f16_gemm_tile(m, n, &bm, &bn);
    if (bm == 128) {
        return launch_f16_gemm_t<128, 128>(w16, x16, y, m, n, k, stream);
    }
    if (bn == 128) {
        return launch_f16_gemm_t<64, 128>(w16, x16, y, m, n, k, stream);
    }
    return launch_f16_gemm_t<64, 64>(w16, x16, y, m, n, k, stream);
}

// ------------------------------------------------- allocation-free variant
// The fp16 activations of q4k_f16_gemm_f32x_noalloc live in this array, one
// copy per device, kept until the process ends.  In host code `scratch` is
// only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) _Float16 scratch[kScratchHalves];

namespace {
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];
std::mutex g_scratch_lock;
}  // namespace

hipError_t f16_scratch(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        return e;
    }
    if (dev < 0 || dev >= kScratchDevices) {
        return hipErrorInvalidDevice;
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lk(g_scratch_lock);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) {
                return e;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace q4k

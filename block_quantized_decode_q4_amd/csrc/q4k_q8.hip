// q4k_q8.hip -- the integer-dot variant: x quantized to Q8 inside the kernel
// and multiplied with the Q4_K codes by int8 dot products (the DP4A GEMV and
// the Q8 quantize kernel that realizar 0.8.5 preloads together,
// src/cuda/executor/layers/modules_utilities.rs, `preload_hw_dp4a_modules`).
//
// Q8 block (the reading taken; the pages name the kernels only): 32
// consecutive elements of x, one Q4_K sub-block; d = amax / 127 in f32, amax
// the largest |x| of the block (NaN when the block holds a NaN); code
// q = nearest-even integer of x * (127 / amax), quotient and product rounded
// to f32; q = 0 where amax is 0 or not a number, or the product is not
// finite.  Its own tolerance: the codes carry x to within d/2 per element
// (plus f32 rounding of the scale), so an output errs by at most
// sum_e |w_e| (d_b(e) / 2 (1 + 2^-20) + 2^-21 |x_e|) from the exact GEMV,
// and the arithmetic after the codes is exact but for the f64 scaling and
// the final rounding to f32.
//
// The GEMV takes kernel 3's layout (q4k_dpp.hip): the line stream of
// q4k_lines.h, lane l = 16 g + j on row j and chunk g of a 16-row tile, the
// 4-bit codes as int8 operands (low nibbles byte & 0x0F, high nibbles
// (byte & 0xF0) ^ 0x80 = 16 q - 128), x shared across the tile's rows by
// DPP row_newbcast folded into the dot instruction.  One code per element
// instead of four digits: 16 dot instructions per step instead of 64, and no
// element needs exact terms, so no lists and no correction branch.
//
// Staged x per superblock column (kQ8Col bytes): four chunks of sixteen
// 4-byte slots (lane j: the codes of code dword j / 2, of the low sub-block
// for even j, the high one for odd j), then per sub-block {d, XI = sum q}.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_device.h"
#include "q4k_kernels.h"
#include "q4k_lines.h"
#include "q4k_xrep.h"

namespace q4k {

constexpr int kQ8Const = 4 * 16 * 4;           // {d, XI} of the eight sub-blocks
constexpr int kQ8Col = kQ8Const + 8 * 8;

// The scale and reciprocal of a block from its largest |x| (NaN if the
// block holds one): d = amax / 127, inv = 127 / amax (0 where amax is 0 or
// NaN), both correctly rounded f32 quotients.
struct Q8Scale {
    float d, inv;
};

__device__ __forceinline__ Q8Scale q8_scale(float amax, bool has_nan)
{
    Q8Scale s;
    const float a = has_nan ? __builtin_nanf("") : amax;
    s.d = a / 127.0f;
    s.inv = a > 0.0f ? 127.0f / a : 0.0f;
    return s;
}

// The code of one element: nearest-even integer of x * inv, 0 if that
// product is not finite.
__device__ __forceinline__ int q8_code(float x, float inv)
{
    const float v = x * inv;
    return __builtin_isfinite(v) ? (int)__builtin_rintf(v) : 0;
}

// Four codes as the bytes of one dword (element 4t + i in byte i)
__device__ __forceinline__ uint32_t q8_pack(int a, int b, int c, int d)
{
    return ((uint32_t)a & 0xFFu) | (((uint32_t)b & 0xFFu) << 8) | (((uint32_t)c & 0xFFu) << 16) |
           ((uint32_t)d << 24);
}

// ------------------------------------------------------------- quantize
// One thread per block of 32 elements of one vector (blocks of all m
// vectors in order); q: m * k codes, d: m * k / 32 scales.
__global__ void __launch_bounds__(256)
q8_quantize_kernel(const float* __restrict__ x, int8_t* __restrict__ q, float* __restrict__ d,
                   int64_t nblocks)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) {
        return;
    }
    const float4* src = reinterpret_cast<const float4*>(x + 32 * b);
    float e[32];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float4 v = src[t];
        e[4 * t] = v.x;
        e[4 * t + 1] = v.y;
        e[4 * t + 2] = v.z;
        e[4 * t + 3] = v.w;
    }
    float amax = 0.f;
    bool has_nan = false;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
        amax = fmaxf(amax, fabsf(e[t]));
        has_nan |= e[t] != e[t];
    }
    const Q8Scale s = q8_scale(amax, has_nan);
    uint4* dst = reinterpret_cast<uint4*>(q + 32 * b);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        uint32_t w4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = 16 * t + 4 * i;
            w4[i] = q8_pack(q8_code(e[o], s.inv), q8_code(e[o + 1], s.inv),
                            q8_code(e[o + 2], s.inv), q8_code(e[o + 3], s.inv));
        }
        dst[t] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    d[b] = s.d;
}

// ---------------------------------------------------------------- GEMV
// One v_dot4c_i32_i8 whose first operand is lane N of the DPP row.
#define Q4K_Q8B(ACC, C, N) \
    "v_dot4c_i32_i8_dpp %" #ACC ", %8, %" #C " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n"
// Code dword u: low codes (operand CL) against the codes of lane NL = 2u into
// accumulator A, high codes (CH) against lane NH = 2u + 1 into A + 4.
#define Q4K_Q8U(A, AH, CL, CH, NL, NH) Q4K_Q8B(A, CL, NL) Q4K_Q8B(AH, CH, NH)

// Sums of one superblock step: t[u % 4] += low codes of dword u times x
// codes, t[4 + u % 4] += high codes times x codes (16 dot products).  As in
// the four-digit kernel, the block keeps its own hazards: two wait states
// before a DPP read of a VALU-written register and five after an EXEC write
// (leading s_nop 4), three before a VALU instruction reads a dot result
// (trailing s_nop 2), and each accumulator is rewritten eight instructions
// after its last write.
__device__ __forceinline__ void q8_dot_step(uint32_t xd, const int (&cl)[8], const int (&ch)[8],
                                            int (&t)[8])
{
    asm("s_nop 4\n"
        Q4K_Q8U(0, 4, 9, 17, 0, 1) Q4K_Q8U(1, 5, 10, 18, 2, 3) Q4K_Q8U(2, 6, 11, 19, 4, 5)
        Q4K_Q8U(3, 7, 12, 20, 6, 7) Q4K_Q8U(0, 4, 13, 21, 8, 9) Q4K_Q8U(1, 5, 14, 22, 10, 11)
        Q4K_Q8U(2, 6, 15, 23, 12, 13) Q4K_Q8U(3, 7, 16, 24, 14, 15)
        "s_nop 2\n"
        : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]),
          "+v"(t[7])
        : "v"(xd),
          "v"(cl[0]), "v"(cl[1]), "v"(cl[2]), "v"(cl[3]), "v"(cl[4]), "v"(cl[5]), "v"(cl[6]),
          "v"(cl[7]),
          "v"(ch[0]), "v"(ch[1]), "v"(ch[2]), "v"(ch[3]), "v"(ch[4]), "v"(ch[5]), "v"(ch[6]),
          "v"(ch[7]));
}

#undef Q4K_Q8U
#undef Q4K_Q8B

// Quantize the 16 consecutive x of group G (column G / 16, elements
// 16 (G % 16) ..) into the column's slots; lanes G and G ^ 1 hold one block
// and meet through DPP (largest |x|, NaN, code sum).  Every lane of the wave
// calls this; `store` is false for groups past the last column.
__device__ __forceinline__ void convert_group_q8(const float4 (&v)[4], int G, bool store,
                                                 unsigned char* xs)
{
    const float e[16] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                         v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
    float amax = 0.f;
    int has_nan = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        amax = fmaxf(amax, fabsf(e[i]));
        has_nan |= e[i] != e[i] ? 1 : 0;
    }
    amax = fmaxf(amax, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                           0, __builtin_bit_cast(int, amax), 0xB1, 0xF, 0xF, false)));   // lane ^ 1
    has_nan |= __builtin_amdgcn_update_dpp(0, has_nan, 0xB1, 0xF, 0xF, false);
    const Q8Scale s = q8_scale(amax, has_nan != 0);
    uint32_t w4[4];
    int xsum = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        w4[t] = q8_pack(q8_code(e[4 * t], s.inv), q8_code(e[4 * t + 1], s.inv),
                        q8_code(e[4 * t + 2], s.inv), q8_code(e[4 * t + 3], s.inv));
        xsum = __builtin_amdgcn_sdot4((int)w4[t], 0x01010101, xsum, false);
    }
    xsum += __builtin_amdgcn_update_dpp(0, xsum, 0xB1, 0xF, 0xF, false);
    if (store) {
        unsigned char* col = xs + (size_t)(G >> 4) * kQ8Col;
        const int e0 = (G & 15) * 16;               // first element within the column
        const int chunk = e0 >> 6;
        const int high = (e0 & 63) >= 32 ? 1 : 0;
        const int u0 = (e0 & 31) >> 2;              // first code dword
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            *reinterpret_cast<uint32_t*>(col + chunk * 64 + (2 * (u0 + t) + high) * 4) = w4[t];
        }
        if ((G & 1) == 0) {
            *reinterpret_cast<uint2*>(col + kQ8Const + ((G & 15) >> 1) * 8) =
                make_uint2(__builtin_bit_cast(uint32_t, s.d), (uint32_t)xsum);
        }
    }
}

// ANY: rows of any whole number of superblocks (line_stream_any); else
// S % 8 == 0 (line_stream).
template <int NW, int XC, bool ANY>
__global__ void __launch_bounds__(NW * 64)
gemv_q8_lines_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x,
                     float* __restrict__ y, int n, int S, int rows_per_block, int slabs_per_task)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ncg = ((S + 7) >> 3) / slabs_per_task;
    constexpr int kWaveRing = ANY ? kRing4Wave : kRingWave;
    (void)wave;

    // LDS: staged x (S columns), the line rings, row sums of slab groups
    const size_t xbytes = (size_t)S * kQ8Col;
    unsigned char* ring = smem + xbytes + wave * kWaveRing;
    double* ypart = reinterpret_cast<double*>(smem + xbytes + NW * kWaveRing);

    // XC groups of 16 x values per thread: all of x when S * 16 <= XC * 64 NW;
    // loads past the end are clamped, their results not stored
    const int ngroups = S * 16;
    float4 xv[XC][4];
    auto issue_x = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int G = min(tid + i * NW * 64, ngroups - 1);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                xv[i][t] = reinterpret_cast<const float4*>(x)[4 * G + t];
            }
        }
    };
    auto convert_x = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int G = tid + i * NW * 64;
            convert_group_q8(xv[i], G, G < ngroups, smem);
        }
    };

    // the lane's (row, chunk) sum over its tasks' superblocks, in f64
    double acc = 0.0;
    const ScaleGather sg = scale_gather(g);
    auto dot_math = [&](const uint4& h, const uint4& q0, const uint4& q1, int c) __attribute__((always_inline)) {
        const unsigned char* col = smem + (size_t)c * kQ8Col;
        const uint32_t xd = *reinterpret_cast<const uint32_t*>(col + g * 64 + j * 4);
        const uint4 k2 = *reinterpret_cast<const uint4*>(col + kQ8Const + g * 16);   // lo, hi {d, XI}
        const uint32_t D[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        int cl[8], ch[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            cl[u] = (int)(D[u] & 0x0F0F0F0Fu);
            ch[u] = (int)((D[u] & 0xF0F0F0F0u) ^ 0x80808080u);
        }
        int t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        q8_dot_step(xd, cl, ch, t);
        const uint32_t sm = gather_scales(h, sg);
        const half2_t dd = __builtin_bit_cast(half2_t, h.x);
        const float d = (float)dd.x;
        const float dmin = (float)dd.y;
        // d sc and dmin m exact in f32, d sc / 16 for the high sub-block whose
        // sums carry 16 q; the integer sums and their products with them are
        // exact in f64, so each sub-block rounds once, at its Q8 scale
        const float Dlo = d * (float)(sm & 0xFFu);
        const float Dhi = d * (float)((sm >> 8) & 0xFFu) * 0.0625f;
        const float Mlo = dmin * (float)((sm >> 16) & 0xFFu);
        const float Mhi = dmin * (float)(sm >> 24);
        const int XIlo = (int)k2.y;
        const int XIhi = (int)k2.w;
        const int Tlo = (t[0] + t[1]) + (t[2] + t[3]);
        const int Thi16 = (t[4] + t[5]) + (t[6] + t[7]) + 128 * XIhi;
        const double rlo = __builtin_fma((double)Dlo, (double)Tlo, -((double)Mlo * (double)XIlo));
        const double rhi = __builtin_fma((double)Dhi, (double)Thi16, -((double)Mhi * (double)XIhi));
        acc = __builtin_fma(rlo, (double)__builtin_bit_cast(float, k2.x), acc);
        acc = __builtin_fma(rhi, (double)__builtin_bit_cast(float, k2.z), acc);
    };
    auto task_end = [&](int task) __attribute__((always_inline)) {
        const int r = (task / ncg) * 16 + j;
        double v = acc;
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (g == 0 && r < rows_here) {
            if (ncg == 1) {
                y[row0 + r] = (float)v;
            } else {
                ypart[(task % ncg) * rows_per_block + r] = v;
            }
        }
        acc = 0.0;
    };
    if constexpr (ANY) {
        constexpr uint32_t kWindow = 511u;
        const uint32_t loff = (uint32_t)(j * 144 * S) & 127u;
        auto step = [&](int c, const unsigned char* rr, uint32_t b0) __attribute__((always_inline)) {
            const uint32_t b = b0 + loff;
            const uint4 h = *reinterpret_cast<const uint4*>(rr + (b & kWindow));
            const uint4 q0 =
                *reinterpret_cast<const uint4*>(rr + ((b + 16u + 32u * (uint32_t)g) & kWindow));
            const uint4 q1 =
                *reinterpret_cast<const uint4*>(rr + ((b + 32u + 32u * (uint32_t)g) & kWindow));
            dot_math(h, q0, q1, c);
        };
        line_stream_any<NW>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                            step, task_end);
    } else {
        const unsigned char* qa[8];
#pragma unroll
        for (int cp = 0; cp < 8; ++cp) {
            qa[cp] = ring + j * kRingRow + ((144u * (uint32_t)cp + 16u + 32u * (uint32_t)g) & 255u);
        }
        auto step = [&](int c, const unsigned char* rr, uint32_t b0) __attribute__((always_inline)) {
            const int cp = (int)(b0 / 144u);         // b0 = 144 cp
            const uint4 h = *reinterpret_cast<const uint4*>(rr + (b0 & 255u));
            const uint4 q0 = *reinterpret_cast<const uint4*>(qa[cp]);
            const uint4 q1 = *reinterpret_cast<const uint4*>(qa[cp] + 16);
            dot_math(h, q0, q1, c);
        };
        line_stream<NW, 3, decltype(issue_x), decltype(convert_x), decltype(step),
                    decltype(task_end), NoSlabFlag, true>(w, x, n, S, rows_per_block,
                                                          slabs_per_task, ring, issue_x,
                                                          convert_x, step, task_end);
    }

    if (ncg > 1) {
        __syncthreads();
        for (int i = tid; i < rows_here; i += NW * 64) {
            double a = 0.0;
            for (int cg = 0; cg < ncg; ++cg) {
                a += ypart[cg * rows_per_block + i];
            }
            y[row0 + i] = (float)a;
        }
    }
}

template <int NW, int XC>
static hipError_t launch_q8_x(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                              hipStream_t stream)
{
    if (p.S % 8 != 0) {
        hipLaunchKernelGGL((gemv_q8_lines_kernel<NW, XC, true>), dim3(p.grid), dim3(NW * 64),
                           p.lds_bytes, stream, w, x, y, p.n, p.S, p.rows_per_block,
                           p.cols_per_task / 8);
    } else {
        hipLaunchKernelGGL((gemv_q8_lines_kernel<NW, XC, false>), dim3(p.grid), dim3(NW * 64),
                           p.lds_bytes, stream, w, x, y, p.n, p.S, p.rows_per_block,
                           p.cols_per_task / 8);
    }
    return hipGetLastError();
}

// XC: groups of 16 x values each thread converts, the power of two covering
// S * 16 / (64 NW), at most 4
template <int NW>
static hipError_t launch_q8_nw(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                               hipStream_t stream)
{
    const int per = (p.S * 16 + NW * 64 - 1) / (NW * 64);
    if (per <= 1) return launch_q8_x<NW, 1>(p, w, x, y, stream);
    if (per <= 2) return launch_q8_x<NW, 2>(p, w, x, y, stream);
    return launch_q8_x<NW, 4>(p, w, x, y, stream);
}

hipError_t launch_gemv_q8(const GemvPlan& p, const void* w, const float* x, float* y,
                          hipStream_t stream)
{
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    if (p.m != 1 || p.S * 16 > 4 * 64 * p.waves_per_block) {
        return hipErrorInvalidValue;
    }
    if (p.waves_per_block == 8) return launch_q8_nw<8>(p, wb, x, y, stream);
    if (p.waves_per_block == 4) return launch_q8_nw<4>(p, wb, x, y, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_quantize_q8(const float* x, int8_t* q, float* d, int64_t nblocks,
                              hipStream_t stream)
{
    const int64_t blocks = (nblocks + 255) / 256;
    hipLaunchKernelGGL(q8_quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, q, d,
                       nblocks);
    return hipGetLastError();
}

size_t q8_lds_bytes(int S, int waves)
{
    return (size_t)S * kQ8Col + (size_t)waves * (S % 8 != 0 ? kRing4Wave : kRingWave);
}

}  // namespace q4k

// q4k_dpp.hip -- Q4_K GEMV for one vector on the vector ALU: the line stream
// of q4k_lines.h feeding integer dot products (v_dot4c_i32_i8), with x
// shared across the 16 rows of a tile by DPP broadcast instead of LDS reads.
//
// Arithmetic (Q4_K superblock format; per sub-block j of 32 weights,
// w = d * sc_j * q - dmin * m_j, so
//   sum_i w_i x_i = d * sc_j * sum_i q_i x_i - dmin * m_j * sum_i x_i):
//  * x is rounded per 32-element sub-block to integers xi = rint(x * 2^s),
//    s chosen so the sub-block's largest |x| * 2^s lies in [2^21, 2^22), and
//    xi is written as three signed base-256 digits D0 + 256 D1 + 65536 D2.
//    Each product's x error is at most 2^-22 of the sub-block's largest |x|.
//  * The 4-bit codes stay packed: for a dword of four code bytes, the low
//    nibbles (byte & 0x0F) and 16 q - 128 for the high nibbles
//    ((byte & 0xF0) ^ 0x80) are signed int8 operands; three v_dot4c_i32_i8
//    per nibble half and dword (one per digit) accumulate exact int32 sums
//    T_d = sum q * D_d.  sum q xi = T_0 + 256 T_1 + 65536 T_2 for the low
//    sub-block; the high one adds 128 * XI (XI = sum xi) and divides by 16.
//  * Superblock scales: fp16 d and dmin and the 6-bit (sc, m) pairs of the
//    lane's two sub-blocks (two byte permutes, gather_scales), applied in
//    f32 once per superblock and lane; the x sums X = 2^-s XI give the min
//    terms, which collect in a second accumulator.
//
// Lane layout of a 16-row tile step (one superblock column): lane l = 16 g +
// j takes row j, chunk g (bytes 16 + 32 g .. of the superblock: elements
// 64 g + i as low nibbles, 64 g + 32 + i as high nibbles).  All 16 lanes of a
// DPP row (the same g) need the same 64 x values.  Each of them reads one 16
// byte slot of the staged x -- lane j holds the three digit dwords of code
// dword u = j / 2, low half (j even) or high half (j odd) -- and the dot
// products take their x operand from lane 2u or 2u + 1 of the row through
// DPP row_newbcast, folded into the dot instruction itself.  So a lane reads
// 16 bytes of x per superblock from LDS, not 192.
//
// Staged x per superblock column (kDotCol bytes): four chunks of sixteen
// 16-byte slots (D0, D1, D2, 0) in the lane order above, then eight
// {2^-s, 8 X} pairs (high sub-blocks keep 2^-s / 16).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_device.h"
#include "q4k_kernels.h"
#include "q4k_lines.h"

namespace q4k {

constexpr int kDotCol = 4 * 16 * 16 + 8 * 8;

// One v_dot4c_i32_i8 whose first operand is lane N of the DPP row.
#define Q4K_DOTB(ACC, X, C, N) \
    "v_dot4c_i32_i8_dpp %" #ACC ", %" #X ", %" #C " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n"
// The six dot products of code dword u: low codes (operand CL) against the
// digits of lane NL = 2u, high codes (CH) against lane NH = 2u + 1.
#define Q4K_DOTU(CL, CH, NL, NH)                                              \
    Q4K_DOTB(0, 6, CL, NL) Q4K_DOTB(1, 7, CL, NL) Q4K_DOTB(2, 8, CL, NL)      \
    Q4K_DOTB(3, 6, CH, NH) Q4K_DOTB(4, 7, CH, NH) Q4K_DOTB(5, 8, CH, NH)

// Digit sums of one superblock step: t[0..2] (low sub-block) and t[3..5]
// (high) += the 48 dot products of the lane's eight code dwords.  The
// compiler does not see the dot instructions inside the block, so the block
// keeps their hazards itself: a DPP operand needs two wait states after a
// VALU write of it and five after a VALU write of EXEC (the leading s_nop),
// and another VALU instruction may read a dot result three wait states
// after the dot at the earliest (the trailing s_nop; without it, waves
// running alone on a SIMD read stale sums).  Within the block each
// accumulator is rewritten six instructions after its last write.
__device__ __forceinline__ void dot_step(const uint4& xd, const int (&cl)[8], const int (&ch)[8],
                                         int (&t)[6])
{
    asm("s_nop 4\n"
        Q4K_DOTU(9, 17, 0, 1) Q4K_DOTU(10, 18, 2, 3) Q4K_DOTU(11, 19, 4, 5)
        Q4K_DOTU(12, 20, 6, 7) Q4K_DOTU(13, 21, 8, 9) Q4K_DOTU(14, 22, 10, 11)
        Q4K_DOTU(15, 23, 12, 13) Q4K_DOTU(16, 24, 14, 15)
        "s_nop 2\n"
        : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5])
        : "v"(xd.x), "v"(xd.y), "v"(xd.z),
          "v"(cl[0]), "v"(cl[1]), "v"(cl[2]), "v"(cl[3]), "v"(cl[4]), "v"(cl[5]), "v"(cl[6]),
          "v"(cl[7]),
          "v"(ch[0]), "v"(ch[1]), "v"(ch[2]), "v"(ch[3]), "v"(ch[4]), "v"(ch[5]), "v"(ch[6]),
          "v"(ch[7]));
}

#undef Q4K_DOTU
#undef Q4K_DOTB

// Scales of chunk g (sub-blocks j = 2g, 2g+1) by two byte gathers with lane
// constants.  With e = 2 (g & 1), P = (s[e], s[e+1], s[e+4], s[e+5]) and
// Q = (s[e+8], s[e+9], s[e+8], s[e+9]):
//   g < 2 : (sc_j, sc_j+1, m_j, m_j+1) = P & 63 (bytewise)
//   g >= 2: the same four from the low and high nibbles of Q (bits 0-3)
//           and bits 6-7 of P (bits 4-5)
// (the 6-bit packing of get_scale_min_k4 in the Q4_K format description).
struct ScaleGather {
    uint32_t selp, selq, ma, mb, mc, md;
};

__device__ __forceinline__ ScaleGather scale_gather(int g)
{
    const uint32_t e = 2u * (uint32_t)(g & 1);
    const bool lo = g < 2;
    ScaleGather s;
    s.selp = e | (e + 1u) << 8 | (e + 4u) << 16 | (e + 5u) << 24;
    s.selq = e | (e + 1u) << 8 | e << 16 | (e + 1u) << 24;
    s.ma = lo ? 0x3F3F3F3Fu : 0u;
    s.mb = lo ? 0u : 0x30303030u;
    s.mc = lo ? 0u : 0x00000F0Fu;
    s.md = lo ? 0u : 0x0F0F0000u;
    return s;
}

// bytes (sc_lo, sc_hi, m_lo, m_hi) of the lane's chunk of header h
__device__ __forceinline__ uint32_t gather_scales(const uint4& h, const ScaleGather& s)
{
    const uint32_t p = __builtin_amdgcn_perm(h.z, h.y, s.selp);   // bytes 0-3: h.y, 4-7: h.z
    const uint32_t q = __builtin_amdgcn_perm(h.w, h.w, s.selq);
    return (p & s.ma) | ((p >> 2) & s.mb) | (q & s.mc) | ((q >> 4) & s.md);
}

// Convert 16 consecutive x values (group G of 16: column G / 16, elements
// 16 (G % 16) ..) into digit slots; lanes G and G ^ 1 hold one sub-block and
// meet through DPP.
__device__ __forceinline__ void convert_group_dot(const float4 (&v)[4], int G, bool store,
                                                  unsigned char* xs)
{
    float mx = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[t].x), fabsf(v[t].y)), fmaxf(fabsf(v[t].z), fabsf(v[t].w))));
    }
    mx = fmaxf(mx, __builtin_bit_cast(float, dpp_i<0xB1>(__builtin_bit_cast(int, mx))));  // lane ^ 1
    int sigma = 0;
    if (mx > 0.f) {
        sigma = 22 - __builtin_amdgcn_frexp_expf(mx);
        sigma = sigma < -126 ? -126 : sigma > 126 ? 126 : sigma;
    }
    const float scale = __builtin_bit_cast(float, (uint32_t)(sigma + 127) << 23);
    // rint(x * 2^s) + 0x808080 as the low bits of x * 2^s + 1.5 * 2^23
    uint32_t usum = 0;
    uint4 dg[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float e[4] = {v[t].x, v[t].y, v[t].z, v[t].w};
        uint32_t u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u[i] = __builtin_bit_cast(uint32_t, __builtin_fmaf(e[i], scale, 12582912.0f)) -
                   0x4ABF7F80u;
            usum += u[i];
        }
        // bytes b of u[0..3] -> digit dword b (balanced: byte ^ 0x80)
        const uint32_t lo01 = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);
        const uint32_t lo23 = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
        const uint32_t hi01 = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);
        const uint32_t hi23 = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
        dg[t] = make_uint4(__builtin_amdgcn_perm(lo23, lo01, 0x05040100u) ^ 0x80808080u,
                           __builtin_amdgcn_perm(lo23, lo01, 0x07060302u) ^ 0x80808080u,
                           __builtin_amdgcn_perm(hi23, hi01, 0x05040100u) ^ 0x80808080u, 0u);
    }
    usum += (uint32_t)dpp_i<0xB1>((int)usum);
    if (store) {
        unsigned char* col = xs + (size_t)(G >> 4) * kDotCol;
        const int e0 = (G & 15) * 16;               // first element within the column
        const int chunk = e0 >> 6;
        const int high = (e0 & 63) >= 32 ? 1 : 0;
        const int u0 = (e0 & 31) >> 2;              // first code dword
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            *reinterpret_cast<uint4*>(col + chunk * 256 + (2 * (u0 + t) + high) * 16) = dg[t];
        }
        if ((G & 1) == 0) {
            const int XI = (int)usum - 32 * 0x808080;
            const float inv = __builtin_bit_cast(float, (uint32_t)(127 - sigma) << 23);
            const int sb = (G & 15) >> 1;
            *reinterpret_cast<float2*>(col + 1024 + sb * 8) =
                make_float2((sb & 1) ? inv * 0.0625f : inv, 8.0f * inv * (float)XI);
        }
    }
}

// ANY: rows of any whole number of superblocks (line_stream_any, four-line
// rings, per-row start offsets); else S % 8 == 0 (line_stream).
template <int NW, int P, int XC, bool ANY>
__global__ void __launch_bounds__(NW * 64)
gemv_dot4_lines_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x,
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

    // LDS: staged x (S columns), the line rings, row sums of slab groups
    const size_t xbytes = (size_t)S * kDotCol;
    unsigned char* ring = smem + xbytes + wave * kWaveRing;
    float* ypart = reinterpret_cast<float*>(smem + xbytes + NW * kWaveRing);

    // XC groups of 16 x values per thread: all of x when S * 16 <= XC * 64 NW;
    // loads past the end are clamped, their results not stored
    const int ngroups = S * 16;
    float4 xv[XC][4];
    auto issue_x = [&]() {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int G = min(tid + i * NW * 64, ngroups - 1);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                xv[i][t] = reinterpret_cast<const float4*>(x)[4 * G + t];
            }
        }
    };
    auto convert_x = [&]() {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int G = tid + i * NW * 64;
            convert_group_dot(xv[i], G, G < ngroups, smem);
        }
    };

    // d terms and 8 x the dmin terms of the lane's (row, chunk) sum
    float acc = 0.f, accm = 0.f;
    const ScaleGather sg = scale_gather(g);
    auto dot_math = [&](const uint4& h, const uint4& q0, const uint4& q1, const unsigned char* col) {
        const uint4 xd = *reinterpret_cast<const uint4*>(col + g * 256 + j * 16);
        const float4 k4 = *reinterpret_cast<const float4*>(col + 1024 + g * 16);
        const uint32_t D[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        int cl[8], ch[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            cl[u] = (int)(D[u] & 0x0F0F0F0Fu);
            ch[u] = (int)((D[u] & 0xF0F0F0F0u) ^ 0x80808080u);
        }
        int t[6] = {0, 0, 0, 0, 0, 0};
        dot_step(xd, cl, ch, t);
        const uint32_t sm = gather_scales(h, sg);
        const half2_t dd = __builtin_bit_cast(half2_t, h.x);
        // low codes q <= 15 and digits |D2| <= 64, |D1|, |D0| <= 128 over 32
        // elements: |T_0 + 256 T_1 + 65536 T_2| < 2^31, exact in int32.  High
        // codes 16 q - 128 take the sum in f32 (T_2 * 65536 exact, |T_2| < 2^19;
        // 256 T_1 + T_0 < 2^27).
        const float tlo = (float)(((t[2] << 8) + t[1]) * 256 + t[0]);
        const float thi = __builtin_fmaf((float)t[5], 65536.0f, (float)(t[4] * 256 + t[3]));
        const float ulo = k4.x * tlo;                         // sum q x, low sub-block
        const float uhi = __builtin_fmaf(k4.z, thi, k4.w);    // sum q x, high sub-block
        acc = __builtin_fmaf((float)dd.x,
                             __builtin_fmaf((float)(sm & 0xFFu), ulo,
                                            (float)((sm >> 8) & 0xFFu) * uhi),
                             acc);
        accm = __builtin_fmaf((float)dd.y,
                              __builtin_fmaf((float)((sm >> 16) & 0xFFu), k4.y,
                                             (float)(sm >> 24) * k4.w),
                              accm);
    };
    auto task_end = [&](int task) {
        const int r = (task / ncg) * 16 + j;
        float v = __builtin_fmaf(-0.125f, accm, acc);
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (g == 0 && r < rows_here) {
            if (ncg == 1) {
                y[row0 + r] = v;
            } else {
                ypart[(task % ncg) * rows_per_block + r] = v;
            }
        }
        acc = 0.f;
        accm = 0.f;
    };
    if constexpr (ANY) {
        // row j starts loff bytes into its first line (tiles start on a
        // line); pieces wrap in the row's four-line window individually
        constexpr uint32_t kWindow = 511u;
        const uint32_t loff = (uint32_t)(j * 144 * S) & 127u;
        auto step = [&](int c, const unsigned char* rr, uint32_t b0) {
            const uint32_t b = b0 + loff;
            const uint4 h = *reinterpret_cast<const uint4*>(rr + (b & kWindow));
            const uint4 q0 =
                *reinterpret_cast<const uint4*>(rr + ((b + 16u + 32u * (uint32_t)g) & kWindow));
            const uint4 q1 =
                *reinterpret_cast<const uint4*>(rr + ((b + 32u + 32u * (uint32_t)g) & kWindow));
            dot_math(h, q0, q1, smem + (size_t)c * kDotCol);
        };
        line_stream_any<NW>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                            step, task_end);
    } else {
        // superblock c' of a slab starts at 144 c' mod 256 in the two-line
        // window of its ring row: the header at that compile-time offset, the
        // lane's 32 code bytes 16 + 32 g further, mod 256 (both 16-byte
        // halves on the same side of the wrap), so their eight addresses are
        // lane constants
        const unsigned char* qa[8];
#pragma unroll
        for (int cp = 0; cp < 8; ++cp) {
            qa[cp] = ring + j * kRingRow + ((144u * (uint32_t)cp + 16u + 32u * (uint32_t)g) & 255u);
        }
        auto step = [&](int c, const unsigned char* rr, uint32_t b0) {
            const int cp = (int)(b0 / 144u);         // b0 = 144 cp
            const uint4 h = *reinterpret_cast<const uint4*>(rr + (b0 & 255u));
            const uint4 q0 = *reinterpret_cast<const uint4*>(qa[cp]);
            const uint4 q1 = *reinterpret_cast<const uint4*>(qa[cp] + 16);
            dot_math(h, q0, q1, smem + (size_t)c * kDotCol);
        };
        line_stream<NW, P>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                           step, task_end);
    }

    if (ncg > 1) {
        __syncthreads();
        for (int i = tid; i < rows_here; i += NW * 64) {
            float a = 0.f;
            for (int cg = 0; cg < ncg; ++cg) {
                a += ypart[cg * rows_per_block + i];
            }
            y[row0 + i] = a;
        }
    }
}

template <int NW, int P, int XC>
static hipError_t launch_dot4_x(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                hipStream_t stream)
{
    if constexpr (P == 3) {
        if (p.S % 8 != 0) {
            hipLaunchKernelGGL((gemv_dot4_lines_kernel<NW, 3, XC, true>), dim3(p.grid),
                               dim3(NW * 64), p.lds_bytes, stream, w, x, y, p.n, p.S,
                               p.rows_per_block, p.cols_per_task / 8);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemv_dot4_lines_kernel<NW, P, XC, false>), dim3(p.grid), dim3(NW * 64),
                       p.lds_bytes, stream, w, x, y, p.n, p.S, p.rows_per_block,
                       p.cols_per_task / 8);
    return hipGetLastError();
}

// XC: groups of 16 x values each thread converts, the power of two covering
// S * 16 / (64 NW), at most 4 (k <= 16384 per 64 NW lanes)
template <int NW, int P>
static hipError_t launch_dot4_p(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                hipStream_t stream)
{
    const int per = (p.S * 16 + NW * 64 - 1) / (NW * 64);
    if (per <= 1) return launch_dot4_x<NW, P, 1>(p, w, x, y, stream);
    if (per <= 2) return launch_dot4_x<NW, P, 2>(p, w, x, y, stream);
    if (per <= 4) return launch_dot4_x<NW, P, 4>(p, w, x, y, stream);
    return hipErrorInvalidValue;
}

template <int NW>
static hipError_t launch_dot4_w(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                hipStream_t stream)
{
    if (p.ring_depth == 9) return launch_dot4_p<NW, 9>(p, w, x, y, stream);
    return launch_dot4_p<NW, 3>(p, w, x, y, stream);
}

hipError_t launch_gemv_dot4(const GemvPlan& p, const void* w, const float* x, float* y,
                            hipStream_t stream)
{
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    switch (p.waves_per_block) {
    case 4: return launch_dot4_w<4>(p, wb, x, y, stream);
    case 8: return launch_dot4_w<8>(p, wb, x, y, stream);
    case 16: return launch_dot4_p<16, 3>(p, wb, x, y, stream);
    default: return hipErrorInvalidValue;
    }
}

size_t dot4_lds_bytes(int S, int waves)
{
    return (size_t)S * kDotCol + (size_t)waves * (S % 8 != 0 ? kRing4Wave : kRingWave);
}

}  // namespace q4k

// q4k_mfma.hip -- Q4_K GEMV for a small batch of vectors (m <= 8; kernels 5
// and 6 up to 16) on the CDNA4 int8 matrix cores, fed by the line stream of
// q4k_lines.h.
//
// With several vectors the same decoded weights meet m different x, which
// makes the multiply a real (small) contraction: the matrix cores take it,
// and the vector ALU keeps the nibble unpack, the header decode and the
// per-superblock scaling.  Two kernels:
//  * gemv_i8_lines_kernel<NW, P, XC, M>: four v_mfma_i32_16x16x64_i8 per
//    superblock and vector (one 16-row tile, one vector per MFMA group);
//    automatic for m = 2.  With m = 1 it runs only when asked for, as the
//    measured matrix-core counterpart of the vector-ALU kernel (q4k_dpp.hip).
//  * gemv_i8_sub_kernel<NW, XC, NQ, false> (kernel 5): one
//    v_mfma_i32_16x16x32_i8 per 32-element sub-block and quad of vectors
//    (up to four quads: one pass over the weights for 16 vectors);
//    automatic for m >= 3.
//  * gemv_i8_sub_kernel<NW, XC, NQ, true> (kernel 6): the same decode with
//    x converted per column by each wave for itself, for batches whose x
//    does not fit the LDS as one stage (m k large).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_device.h"
#include "q4k_kernels.h"
#include "q4k_lines.h"

namespace q4k {


// ---------------------------------------------------------------------------
// int8 matrix-core decode (v_mfma_i32_16x16x64_i8).
//
// Operands of one MFMA (16 x 16 x 64): lane l = 16 g + j holds
//   A[i = j][k = 16g .. 16g+15] (16 bytes), B[k = 16g .. 16g+15][j], D[4g + r][j].
//
//  * B = codes of 16 weight rows (j = row).  Lane group g reads chunk g of its
//    row (32 code bytes: sub-block 2g in the low nibbles, 2g+1 in the high
//    ones).  Low codes: byte & 0x0F (one AND per four codes).  High codes:
//    (byte & 0xF0) ^ 0x80 = 16 q - 128 as a signed byte (one three-input
//    bit operation per four codes); the -128 is undone with the sub-block's
//    integer x sum.  Four MFMAs per superblock: bytes 0-15 and 16-31 of the
//    chunk, low and high codes.
//  * A = x as a 23-bit integer per element, xi = rint(x * 2^sigma_s) with one
//    power of two per 32-element sub-block s (largest |x| in [2^21, 2^22)),
//    split into three signed base-256 digits xi = l0 + 256 l1 + 65536 l2.
//    Row i = 4g' + l of A holds digit l of sub-block 2g' (low MFMAs) or
//    2g'+1 (high MFMAs) in k-group g', zero elsewhere, so D rows 4g..4g+2 of
//    lane (g, j) are the three digit dot products of exactly the two
//    sub-blocks whose scales lane (g, j) decodes.  The zero rows cost
//    nothing: inactive lanes read a zero slot of the stage.
//  * Per step and lane: T = D0 + 256 D1 + 65536 D2 (exact in int32 up to the
//    last f32 rounding), then
//      acc += d * (sc_lo * 2^-sigma_lo * T_lo
//                  + sc_hi * (2^-sigma_hi / 16 * T_hi + 8 * X_hi))
//             - dmin * (m_lo * X_lo + m_hi * X_hi)
//    with X = 2^-sigma * XI the sum of the quantized x of a sub-block (XI
//    its integer sum).
//  * Quantizing x to 23 bits per sub-block bounds the error of a product by
//    2^-22 of the sub-block's largest |x| times |w|.
// ---------------------------------------------------------------------------

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kI8MuBytes = 208;                 // 12 digit slots of 16 B + a zero slot
constexpr int kI8ZeroSlot = 192;
constexpr int kI8ColA = 4 * kI8MuBytes;         // four MFMA operands per column
constexpr int kI8ColConst = 4 * 32;             // eight floats per lane group
constexpr int kI8ColBytes = kI8ColA + kI8ColConst;

// Convert four (column, vector) pairs at once, one per 16-lane group: lane
// l takes elements 16 (l % 16) .. 16 (l % 16) + 15 of its pair, half of a
// sub-block, so each lane writes three whole 16-byte digit slots and the
// per-lane costs (largest |x|, scale, sums) are shared by 16 elements.
// `col` is the LDS slot of the lane's pair: 12 digit slots of 16 bytes per
// MFMA operand mu (digit l of the 16 elements of k-group g at slot 3 g + l,
// a zero slot after them) and the constants {2^-s, 2^-s / 16, 8 X, X_lo,
// X_hi} of each lane group's two sub-blocks.
__device__ __forceinline__ void convert4_i8(const float4 (&v)[4], unsigned char* col, int lane)
{
    const int le = lane & 15;
    const int s = le >> 1;                    // sub-block
    const int half = le & 1;                  // its elements 0-15 or 16-31
    const int g = s >> 1;
    const int mu = 2 * (s & 1) + half;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    m = fmaxf(m, __builtin_bit_cast(float, dpp_i<0xB1>(__builtin_bit_cast(int, m))));  // lane l ^ 1
    int sigma = 0;
    if (m > 0.f) {
        sigma = 22 - __builtin_amdgcn_frexp_expf(m);
        sigma = sigma < -126 ? -126 : sigma > 126 ? 126 : sigma;
    }
    const float scale = __builtin_bit_cast(float, (uint32_t)(sigma + 127) << 23);
    uint32_t usum = 0;
    uint4 dig[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float vals[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u[t] = __builtin_bit_cast(uint32_t, __builtin_fmaf(vals[t], scale, 12582912.0f)) -
                   0x4ABF7F80u;
            usum += u[t];
        }
        const uint32_t lo01 = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);
        const uint32_t lo23 = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
        const uint32_t hi01 = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);
        const uint32_t hi23 = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
        const uint32_t d0 = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u) ^ 0x80808080u;
        const uint32_t d1 = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u) ^ 0x80808080u;
        const uint32_t d2 = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u) ^ 0x80808080u;
        (&dig[0].x)[i] = d0;
        (&dig[1].x)[i] = d1;
        (&dig[2].x)[i] = d2;
    }
    unsigned char* slot = col + mu * kI8MuBytes + g * 48;
    *reinterpret_cast<uint4*>(slot) = dig[0];
    *reinterpret_cast<uint4*>(slot + 16) = dig[1];
    *reinterpret_cast<uint4*>(slot + 32) = dig[2];
    if (le < 4) {
        *reinterpret_cast<uint4*>(col + le * kI8MuBytes + kI8ZeroSlot) = make_uint4(0, 0, 0, 0);
    }
    const uint32_t us2 = usum + (uint32_t)dpp_i<0xB1>((int)usum);
    const int XI = (int)us2 - 32 * 0x808080;
    if (half == 0) {
        float* c = reinterpret_cast<float*>(col + kI8ColA + g * 32);
        const float inv = __builtin_bit_cast(float, (uint32_t)(127 - sigma) << 23);
        const float xq = inv * (float)XI;
        if ((s & 1) == 0) {
            c[0] = inv;
            c[3] = xq;
        } else {
            c[1] = inv * 0.0625f;
            c[2] = 8.0f * xq;
            c[4] = xq;
        }
    }
}

// The 16 x elements lane l converts in convert4_i8, of pair p (column p / m
// of vector p % m).
__device__ __forceinline__ void load_x_quarter(const float* __restrict__ x, int k, int m, int p,
                                               int lane, float4 (&v)[4])
{
    const float* src = x + (size_t)(p % m) * k + (size_t)(p / m) * 256 + 16 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = reinterpret_cast<const float4*>(src)[i];
    }
}

struct TileI8 {
    uint4 h;       // the lane's row header
    uint4 q0, q1;  // chunk g of the row: code bytes 0-15 and 16-31
};

struct ColI8 {
    i32x4_t a[4];     // MFMA A operands of the column
    float c0, c1, c2, xlo, xhi;
};

__device__ __forceinline__ ColI8 read_col_i8(const unsigned char* col, uint32_t a_off, int g)
{
    ColI8 c;
#pragma unroll
    for (int mu = 0; mu < 4; ++mu) {
        c.a[mu] = *reinterpret_cast<const i32x4_t*>(col + a_off + mu * kI8MuBytes);
    }
    const float4 k = *reinterpret_cast<const float4*>(col + kI8ColA + g * 32);
    c.c0 = k.x;
    c.c1 = k.y;
    c.c2 = k.z;
    c.xlo = k.w;
    c.xhi = *reinterpret_cast<const float*>(col + kI8ColA + g * 32 + 16);
    return c;
}

__device__ __forceinline__ i32x4_t lo_codes(const uint4& q)
{
    return i32x4_t{(int)(q.x & 0x0F0F0F0Fu), (int)(q.y & 0x0F0F0F0Fu), (int)(q.z & 0x0F0F0F0Fu),
                   (int)(q.w & 0x0F0F0F0Fu)};
}

__device__ __forceinline__ i32x4_t hi_codes(const uint4& q)
{
    return i32x4_t{(int)((q.x & 0xF0F0F0F0u) ^ 0x80808080u), (int)((q.y & 0xF0F0F0F0u) ^ 0x80808080u),
                   (int)((q.z & 0xF0F0F0F0u) ^ 0x80808080u), (int)((q.w & 0xF0F0F0F0u) ^ 0x80808080u)};
}

__device__ __forceinline__ float digits_value(const i32x4_t& D)
{
    return __builtin_fmaf((float)D[2], 65536.0f, (float)(D[1] * 256 + D[0]));
}

// The weight side of one (tile, column) step: unpacked codes and the
// lane's chunk scales, shared by every vector.
struct StepW {
    i32x4_t lo0, lo1, hi0, hi1;
    ChunkScalesD s;
};

__device__ __forceinline__ StepW step_weights(const TileI8& cur, uint32_t sh, uint32_t sel)
{
    StepW t;
    t.lo0 = lo_codes(cur.q0);
    t.lo1 = lo_codes(cur.q1);
    t.hi0 = hi_codes(cur.q0);
    t.hi1 = hi_codes(cur.q1);
    t.s = decode_chunk(cur.h, sh, sel);
    return t;
}

// One vector's part of a step: four MFMAs and the scaling; the lane's
// partial of its row.
__device__ __forceinline__ float step_vector(const StepW& t, const ColI8& col)
{
    const i32x4_t zero = {0, 0, 0, 0};
    i32x4_t Dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(col.a[0], t.lo0, zero, 0, 0, 0);
    Dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(col.a[1], t.lo1, Dl, 0, 0, 0);
    i32x4_t Dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(col.a[2], t.hi0, zero, 0, 0, 0);
    Dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(col.a[3], t.hi1, Dh, 0, 0, 0);
    const float u_lo = col.c0 * digits_value(Dl);
    const float u_hi = __builtin_fmaf(col.c1, digits_value(Dh), col.c2);
    float t1 = t.s.sc_lo * u_lo;
    t1 = __builtin_fmaf(t.s.sc_hi, u_hi, t1);
    float t2 = t.s.m_lo * col.xlo;
    t2 = __builtin_fmaf(t.s.m_hi, col.xhi, t2);
    return __builtin_fmaf(-t.s.dmin, t2, t.s.d * t1);
}

// ---------------------------------------------------------------------------
// Line-streamed int8 matrix-core kernel (rows of whole 128-byte lines).
//
// The operands and arithmetic above, fed by the line stream of q4k_lines.h:
// whole 128-byte lines per row into a per-wave LDS ring, from which the
// lanes read the tile layout of the matrix cores; M vectors share the
// weight side (codes, scales) of each step.
// ---------------------------------------------------------------------------

template <int NW, int P, int XC, int M>
__global__ void __launch_bounds__(NW * 64)
gemv_i8_lines_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x,
                     float* __restrict__ y, int n, int S, int rows_per_block, int slabs_per_task)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    const bool active = (j >> 2) == g && (j & 3) < 3;
    const uint32_t a_off = active ? (uint32_t)((g * 3 + (j & 3)) * 16) : (uint32_t)kI8ZeroSlot;
    const uint32_t sh = (uint32_t)(g & 1) * 16u;
    const uint32_t sel = g < 2 ? 0xFFFFFFFFu : 0u;
    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ncg = (S >> 3) / slabs_per_task;

    // LDS: staged x (S columns of M vectors, column-major, and a spare
    // slot), the line rings, row sums
    const int npairs = S * M;
    const size_t xbytes = (size_t)(npairs + 1) * kI8ColBytes;
    unsigned char* ring = smem + xbytes + wave * kRingWave;
    float* ypart = reinterpret_cast<float*>(smem + xbytes + NW * kRingWave);
    const int k = S * 256;

    // XC groups of four (column, vector) pairs of x per wave, one pair per
    // 16-lane group: all of them when S * M <= 4 * XC * NW; pair p is column
    // p / M of vector p % M
    float4 xv[XC][4];
    auto issue_x = [&]() {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int pr = min(4 * (wave + i * NW) + (lane >> 4), npairs - 1);
            load_x_quarter(x, k, M, pr, lane, xv[i]);
        }
    };
    // unconditional conversions (a load feeding a conditional use would be
    // sunk into the branch and wait for every load before it); pairs past
    // the last go to a spare slot
    auto convert_x = [&]() {
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int pr = min(4 * (wave + i * NW) + (lane >> 4), npairs);
            convert4_i8(xv[i], smem + (size_t)pr * kI8ColBytes, lane);
        }
        for (int q = XC * NW + wave; 4 * q < npairs; q += NW) {
            const int pr = min(4 * q + (lane >> 4), npairs - 1);
            float4 v[4];
            load_x_quarter(x, k, M, pr, lane, v);
            convert4_i8(v, smem + (size_t)(4 * q + (lane >> 4) < npairs ? pr : npairs) * kI8ColBytes,
                        lane);
        }
    };

    float acc[M];
#pragma unroll
    for (int b = 0; b < M; ++b) {
        acc[b] = 0.f;
    }
    auto step = [&](int c, const unsigned char* rr, uint32_t b0) {
        TileI8 t;
        t.h = *reinterpret_cast<const uint4*>(rr + (b0 & 255u));
        t.q0 = *reinterpret_cast<const uint4*>(rr + ((b0 + 16u + 32u * (uint32_t)g) & 255u));
        t.q1 = *reinterpret_cast<const uint4*>(rr + ((b0 + 32u + 32u * (uint32_t)g) & 255u));
        const StepW sw = step_weights(t, sh, sel);
#pragma unroll
        for (int b = 0; b < M; ++b) {
            const ColI8 col = read_col_i8(smem + (size_t)(c * M + b) * kI8ColBytes, a_off, g);
            acc[b] += step_vector(sw, col);
        }
    };
    auto task_end = [&](int task) {
        const int r = (task / ncg) * 16 + j;
#pragma unroll
        for (int b = 0; b < M; ++b) {
            float v = acc[b];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (g == 0 && r < rows_here) {
                if (ncg == 1) {
                    y[(size_t)b * n + row0 + r] = v;
                } else {
                    ypart[(b * ncg + task % ncg) * rows_per_block + r] = v;
                }
            }
            acc[b] = 0.f;
        }
    };
    line_stream<NW, P>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x, step,
                       task_end);

    if (ncg > 1) {
        __syncthreads();
        for (int i = tid; i < rows_here * M; i += NW * 64) {
            const int b = i / rows_here;
            const int r = i - b * rows_here;
            float a = 0.f;
            for (int cg = 0; cg < ncg; ++cg) {
                a += ypart[(b * ncg + cg) * rows_per_block + r];
            }
            y[(size_t)b * n + row0 + r] = a;
        }
    }
}

// ---------------------------------------------------------------------------
// Sub-block int8 matrix-core kernel for several vectors
// (v_mfma_i32_16x16x32_i8, line-streamed weights).
//
// Operands of one MFMA (16 x 16 x 32): lane l = 16 g + j holds
//   A[i = j][k = 8g .. 8g+7] (8 bytes), B[k = 8g .. 8g+7][j], D[4g + r][j].
//
// One MFMA covers one 32-element sub-block s for four vectors: B = the codes
// of sub-block s of the 16 rows of the tile (lane group g: elements 8g ..
// 8g+7, taken from bytes 8g .. 8g+7 of the chunk, low or high nibbles as in
// the kernels above), A row 4 b' + l = digit l of vector b' of the quad (row
// 4 b' + 3 zero).  A is dense, so a superblock costs eight small MFMAs per
// quad of vectors instead of four large ones per vector, and lane (g, j) ends
// with the three digit sums of vector g of the quad for row j: it needs no
// other lane, but it scales all eight sub-blocks of its row:
//   acc += d * sum_s sc_s * u_s - dmin * sum_s m_s * X_s,
//   u_s = 2^-sigma_s * T_s (low sub-blocks), 2^-sigma_s / 16 * T_s + 8 X_s (high),
// T = D0 + 256 D1 + 65536 D2, X_s the quantized x sum of the sub-block.
// ---------------------------------------------------------------------------

constexpr int kSbBlock = 49 * 8;              // 48 digit slots of 8 bytes and a zero slot
constexpr int kSbZero = 48 * 8;
constexpr int kSbQuad = 8 * kSbBlock;         // A operands of one column and vector quad
constexpr int kSbConst = 8 * 8;               // {scale, X} of the eight sub-blocks of one vector
constexpr int kSbGroup = kSbQuad + 4 * kSbConst;   // one column, one quad: A, then constants

// Convert one (column, vector quad): lane l takes vector l / 16 of the quad
// and elements 16 (l % 16) .. +15 of the column (half of sub-block (l % 16) /
// 2).  Digits as in convert4_i8; here digit l of elements 8g .. 8g+7 of
// sub-block s of vector b' goes to slot (g, b', l) of block s.
__device__ __forceinline__ void convert4_sb(const float4 (&v)[4], unsigned char* grp, int lane)
{
    const int le = lane & 15;
    const int bq = lane >> 4;                 // vector within the quad
    const int s = le >> 1;                    // sub-block
    const int half = le & 1;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    }
    m = fmaxf(m, __builtin_bit_cast(float, dpp_i<0xB1>(__builtin_bit_cast(int, m))));  // lane l ^ 1
    int sigma = 0;
    if (m > 0.f) {
        sigma = 22 - __builtin_amdgcn_frexp_expf(m);
        sigma = sigma < -126 ? -126 : sigma > 126 ? 126 : sigma;
    }
    const float scale = __builtin_bit_cast(float, (uint32_t)(sigma + 127) << 23);
    uint32_t usum = 0;
    uint32_t dig[3][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float vals[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
        uint32_t u[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u[t] = __builtin_bit_cast(uint32_t, __builtin_fmaf(vals[t], scale, 12582912.0f)) -
                   0x4ABF7F80u;
            usum += u[t];
        }
        const uint32_t lo01 = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);
        const uint32_t lo23 = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
        const uint32_t hi01 = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);
        const uint32_t hi23 = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
        dig[0][i] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u) ^ 0x80808080u;
        dig[1][i] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u) ^ 0x80808080u;
        dig[2][i] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u) ^ 0x80808080u;
    }
    unsigned char* blk = grp + s * kSbBlock;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int gk = 2 * half + h;          // k-group of these eight elements
#pragma unroll
        for (int l = 0; l < 3; ++l) {
            *reinterpret_cast<uint2*>(blk + ((gk * 4 + bq) * 3 + l) * 8) =
                make_uint2(dig[l][2 * h], dig[l][2 * h + 1]);
        }
    }
    // the zero slot and the sub-block constants: every lane of a pair holds
    // the same values (pair max and sum by DPP), so both store them -- no
    // branch inside the callers' unrolled loops
    *reinterpret_cast<uint2*>(blk + kSbZero) = make_uint2(0, 0);
    const uint32_t us2 = usum + (uint32_t)dpp_i<0xB1>((int)usum);
    const int XI = (int)us2 - 32 * 0x808080;
    const float inv = __builtin_bit_cast(float, (uint32_t)(127 - sigma) << 23);
    *reinterpret_cast<float2*>(grp + kSbQuad + bq * kSbConst + s * 8) =
        make_float2((s & 1) ? inv * 0.0625f : inv, inv * (float)XI);
}

// The eight sub-block scales and mins of a header as floats.
struct RowScales {
    float d, dmin;
    float sc[8], m[8];
};

__device__ __forceinline__ RowScales decode_row(const uint4& h)
{
    RowScales r;
    const half2_t dd = __builtin_bit_cast(half2_t, h.x);
    r.d = (float)dd.x;
    r.dmin = (float)dd.y;
    const uint32_t sc03 = h.y & 0x3F3F3F3Fu;
    const uint32_t m03 = h.z & 0x3F3F3F3Fu;
    const uint32_t sc47 = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t m47 = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        r.sc[b] = (float)((sc03 >> (8 * b)) & 0xFFu);
        r.m[b] = (float)((m03 >> (8 * b)) & 0xFFu);
        r.sc[4 + b] = (float)((sc47 >> (8 * b)) & 0xFFu);
        r.m[4 + b] = (float)((m47 >> (8 * b)) & 0xFFu);
    }
    return r;
}

// Columns of x a wave of kernel 6 holds in registers ahead of its step: with
// four, waiting for a column's x (loads complete in order) never waits for
// a weight line before the line stream itself would (the lines are three
// ahead); two vector quads take two, as 4 x 32 registers do not fit, and
// four quads one (64 registers).
template <int NQ>
constexpr int jit_ahead()
{
    return NQ == 1 ? 4 : NQ == 2 ? 2 : 1;
}

// JIT = false (kernel 5): x staged whole in LDS before the stream.  JIT =
// true (kernel 6): each wave converts the x column of each of its steps for
// itself into its own LDS groups, from registers loaded jit_ahead columns
// earlier -- for batches whose whole x stage does not fit the LDS.
// ANY: rows of any whole number of superblocks (line_stream_any: four-line
// rings, per-row start offsets); else S % 8 == 0 (line_stream).
template <int NW, int XC, int NQ, bool JIT, bool ANY>
__global__ void __launch_bounds__(NW * 64)
gemv_i8_sub_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x,
                   float* __restrict__ y, int n, int S, int m, int rows_per_block,
                   int slabs_per_task)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int j = lane & 15;
    // A row of this lane: vector j / 4 of the quad, digit j % 4 (3: zero)
    const uint32_t a_off = (j & 3) < 3 ? (uint32_t)(((g * 4 + (j >> 2)) * 3 + (j & 3)) * 8)
                                       : (uint32_t)kSbZero;
    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ncg = ((S + 7) >> 3) / slabs_per_task;
    const int k = S * 256;
    constexpr int kWaveRing = ANY ? kRing4Wave : kRingWave;
    constexpr uint32_t kWindow = ANY ? 511u : 255u;        // ring window of a row, minus one
    // byte offset of the lane's row within its first line (tiles start on a line)
    const uint32_t loff = ANY ? (uint32_t)(j * 144 * S) & 127u : 0u;

    // LDS: staged x (S columns x NQ quads and a spare group; JIT: NQ groups
    // per wave), the line rings, row sums
    const int ngroups = S * NQ;
    const size_t xbytes = JIT ? (size_t)NW * NQ * kSbGroup : (size_t)(ngroups + 1) * kSbGroup;
    unsigned char* xw = smem + (JIT ? (size_t)wave * NQ * kSbGroup : 0);
    unsigned char* ring = smem + xbytes + wave * kWaveRing;
    float* ypart = reinterpret_cast<float*>(smem + xbytes + NW * kWaveRing);

    // group q0 = column q0 / NQ, quad q0 % NQ; 16-lane group l / 16 takes
    // vector 4 (q0 % NQ) + l / 16 (past the last vector the last vector
    // again: its digits reach only the D rows of lanes whose sums are never
    // stored, so they need no zeroing)
    float4 xv[XC][4];
    auto load_group = [&](int q0, float4 (&v)[4]) {
        const int qc = min(q0, ngroups - 1);
        const int b = 4 * (qc % NQ) + (lane >> 4);
        const float* src = x + (size_t)min(b, m - 1) * k + (size_t)(qc / NQ) * 256 + 16 * (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = reinterpret_cast<const float4*>(src)[i];
        }
    };
    // JIT: slot a holds the x of a column with c mod kA = a (first column
    // of the wave's first slab: c_first)
    constexpr int kA = JIT ? jit_ahead<NQ>() : 1;
    float4 xa[kA][NQ][4];
    const int ntasks = ((rows_here + 15) >> 4) * ncg;
    const int c_first = 8 * ((min(wave, ntasks - 1) % ncg) * slabs_per_task);
    auto issue_x = [&]() {
        if constexpr (JIT) {
#pragma unroll
            for (int a = 0; a < kA; ++a) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    load_group((c_first + a) * NQ + q, xa[a][q]);
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            load_group(wave + i * NW, xv[i]);
        }
    };
    auto convert_x = [&]() {
        if constexpr (JIT) {
            return;
        }
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int q0 = wave + i * NW;
            convert4_sb(xv[i], smem + (size_t)min(q0, ngroups) * kSbGroup, lane);
        }
        for (int q0 = XC * NW + wave; q0 < ngroups; q0 += NW) {
            float4 v[4];
            load_group(q0, v);
            convert4_sb(v, smem + (size_t)q0 * kSbGroup, lane);
        }
    };

    float acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        acc[q] = 0.f;
    }
    // one superblock of the lane's tile (ring row rr, offset b0) against
    // the x groups of its column at grp0, grp0 + kSbGroup, ...
    auto decode = [&](const unsigned char* rr, uint32_t b0, const unsigned char* grp0) {
        const uint32_t b = b0 + loff;
        const uint4 hdr = *reinterpret_cast<const uint4*>(rr + (b & kWindow));
        uint2 raw[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            raw[cc] = *reinterpret_cast<const uint2*>(rr + ((b + 16u + 32u * cc + 8u * g) & kWindow));
        }
        long codes[8];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            codes[2 * cc] = __builtin_bit_cast(long, make_uint2(raw[cc].x & 0x0F0F0F0Fu,
                                                                 raw[cc].y & 0x0F0F0F0Fu));
            codes[2 * cc + 1] = __builtin_bit_cast(
                long, make_uint2((raw[cc].x & 0xF0F0F0F0u) ^ 0x80808080u,
                                 (raw[cc].y & 0xF0F0F0F0u) ^ 0x80808080u));
        }
        const RowScales rs = decode_row(hdr);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const unsigned char* grp = grp0 + (size_t)q * kSbGroup;
            const float4* cst = reinterpret_cast<const float4*>(grp + kSbQuad + g * kSbConst);
            float t1 = 0.f, t2 = 0.f;
#pragma unroll
            for (int sp = 0; sp < 4; ++sp) {
                const float4 k2 = cst[sp];        // {scale, X} of sub-blocks 2sp, 2sp+1
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int sb = 2 * sp + h;
                    const long a = *reinterpret_cast<const long*>(grp + sb * kSbBlock + a_off);
                    const i32x4_t zero = {0, 0, 0, 0};
                    const i32x4_t D = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, codes[sb], zero, 0, 0, 0);
                    const float T = digits_value(D);
                    const float sca = h ? k2.z : k2.x;
                    const float X = h ? k2.w : k2.y;
                    const float u = h ? __builtin_fmaf(sca, T, 8.0f * X) : sca * T;
                    t1 = __builtin_fmaf(rs.sc[sb], u, t1);
                    t2 = __builtin_fmaf(rs.m[sb], X, t2);
                }
            }
            acc[q] = __builtin_fmaf(rs.d, t1, acc[q]);
            acc[q] = __builtin_fmaf(-rs.dmin, t2, acc[q]);
        }
    };
    auto step = [&](int c, const unsigned char* rr, uint32_t b0) {
        decode(rr, b0, smem + (size_t)c * NQ * kSbGroup);
    };
    // JIT: convert column c (slot cp mod kA) into the wave's groups, refill
    // the slot with the column kA positions on (past cend: the next slab's or
    // task's, from cn), then decode; the groups are rewritten only after this
    // step's reads of them (the wave's LDS accesses complete in order).
    // Positions past a partial slab's end (invalid) keep the slots cycling.
    auto step_jit = [&](int c, int cend, int cn, const unsigned char* rr, uint32_t b0, int cp,
                        bool valid) {
        float4 (&v)[NQ][4] = xa[JIT ? cp % kA : 0];
        __builtin_amdgcn_sched_barrier(0);
        if (valid) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                convert4_sb(v[q], xw + (size_t)q * kSbGroup, lane);
            }
        }
        const int ca = c + kA < cend ? c + kA : cn + (c + kA - cend);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            load_group(ca * NQ + q, v[q]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (valid) {
            decode(rr, b0, xw);
        }
    };
    auto task_end = [&](int task) {
        const int r = (task / ncg) * 16 + j;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int b = 4 * q + g;
            if (b < m && r < rows_here) {
                if (ncg == 1) {
                    y[(size_t)b * n + row0 + r] = acc[q];
                } else {
                    ypart[(b * ncg + task % ncg) * rows_per_block + r] = acc[q];
                }
            }
            acc[q] = 0.f;
        }
    };
    if constexpr (JIT && ANY) {
        line_stream_any<NW>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                            step_jit, task_end);
    } else if constexpr (JIT) {
        line_stream<NW, 3>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                           step_jit, task_end);
    } else if constexpr (ANY) {
        line_stream_any<NW>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                            step, task_end);
    } else {
        line_stream<NW, 3>(w, x, n, S, rows_per_block, slabs_per_task, ring, issue_x, convert_x,
                           step, task_end);
    }

    if (ncg > 1) {
        __syncthreads();
        for (int i = tid; i < rows_here * m; i += NW * 64) {
            const int b = i / rows_here;
            const int r = i - b * rows_here;
            float a = 0.f;
            for (int cg = 0; cg < ncg; ++cg) {
                a += ypart[(b * ncg + cg) * rows_per_block + r];
            }
            y[(size_t)b * n + row0 + r] = a;
        }
    }
}

template <int XC, int NQ, bool JIT = false>
static hipError_t launch_sub_x(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                               hipStream_t stream)
{
    if (p.S % 8 != 0) {
        hipLaunchKernelGGL((gemv_i8_sub_kernel<8, XC, NQ, JIT, true>), dim3(p.grid), dim3(512),
                           p.lds_bytes, stream, w, x, y, p.n, p.S, p.m, p.rows_per_block,
                           p.cols_per_task / 8);
    } else {
        hipLaunchKernelGGL((gemv_i8_sub_kernel<8, XC, NQ, JIT, false>), dim3(p.grid), dim3(512),
                           p.lds_bytes, stream, w, x, y, p.n, p.S, p.m, p.rows_per_block,
                           p.cols_per_task / 8);
    }
    return hipGetLastError();
}

// (column, quad) groups each of the eight waves converts before the first
// barrier: the power of two covering S * NQ / 8, at most 4
template <int NQ>
static hipError_t launch_sub(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                             hipStream_t stream)
{
    const int per = (p.S * NQ + 7) / 8;
    if (per <= 1) return launch_sub_x<1, NQ>(p, w, x, y, stream);
    if (per <= 2) return launch_sub_x<2, NQ>(p, w, x, y, stream);
    return launch_sub_x<4, NQ>(p, w, x, y, stream);
}

template <int NW, int P, int XC, int M>
static hipError_t launch_lines_x(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                 hipStream_t stream)
{
    hipLaunchKernelGGL((gemv_i8_lines_kernel<NW, P, XC, M>), dim3(p.grid), dim3(NW * 64),
                       p.lds_bytes, stream, w, x, y, p.n, p.S, p.rows_per_block,
                       p.cols_per_task / 8);
    return hipGetLastError();
}

// groups of four (column, vector) pairs of x each wave converts before the
// first barrier: the power of two covering S * m / (4 NW), at most 4 (the
// rest follow in a loop)
template <int NW, int P>
static hipError_t launch_lines_p(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                 hipStream_t stream)
{
    const int per = (p.S + 4 * NW - 1) / (4 * NW);
    if (per <= 1) return launch_lines_x<NW, P, 1, 1>(p, w, x, y, stream);
    if (per <= 2) return launch_lines_x<NW, P, 2, 1>(p, w, x, y, stream);
    return launch_lines_x<NW, P, 4, 1>(p, w, x, y, stream);
}

template <int NW>
static hipError_t launch_lines(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                               hipStream_t stream)
{
    if (p.ring_depth == 9) return launch_lines_p<NW, 9>(p, w, x, y, stream);
    return launch_lines_p<NW, 3>(p, w, x, y, stream);
}

// several vectors: eight waves, three lines in flight
template <int M>
static hipError_t launch_lines_m(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                                 hipStream_t stream)
{
    const int per = (p.S * M + 31) / 32;
    if (per <= 1) return launch_lines_x<8, 3, 1, M>(p, w, x, y, stream);
    if (per <= 2) return launch_lines_x<8, 3, 2, M>(p, w, x, y, stream);
    return launch_lines_x<8, 3, 4, M>(p, w, x, y, stream);
}

// vector quads of the sub-block kernels' launch for m vectors (1, 2 or 4)
static int sub_quads(int m)
{
    return m > 8 ? 4 : m > 4 ? 2 : 1;
}

hipError_t launch_gemv_mfma(const GemvPlan& p, const void* w, const float* x, float* y,
                            hipStream_t stream)
{
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    if (p.kernel == 5 || p.kernel == 6) {
        const int nq = sub_quads(p.m);         // the quads sub_lds_bytes, jit_lds_bytes size
        if (p.kernel == 5) {
            if (nq == 4) return launch_sub<4>(p, wb, x, y, stream);
            if (nq == 2) return launch_sub<2>(p, wb, x, y, stream);
            return launch_sub<1>(p, wb, x, y, stream);
        }
        if (nq == 4) return launch_sub_x<1, 4, true>(p, wb, x, y, stream);
        if (nq == 2) return launch_sub_x<1, 2, true>(p, wb, x, y, stream);
        return launch_sub_x<1, 1, true>(p, wb, x, y, stream);
    }
    switch (p.m) {
    case 1: break;
    case 2: return launch_lines_m<2>(p, wb, x, y, stream);
    case 3: return launch_lines_m<3>(p, wb, x, y, stream);
    case 4: return launch_lines_m<4>(p, wb, x, y, stream);
    case 5: return launch_lines_m<5>(p, wb, x, y, stream);
    case 6: return launch_lines_m<6>(p, wb, x, y, stream);
    case 7: return launch_lines_m<7>(p, wb, x, y, stream);
    default: return launch_lines_m<8>(p, wb, x, y, stream);
    }
    if (p.waves_per_block == 8) return launch_lines<8>(p, wb, x, y, stream);
    if (p.waves_per_block == 16) return launch_lines_p<16, 3>(p, wb, x, y, stream);
    return launch_lines<4>(p, wb, x, y, stream);
}

size_t sub_lds_bytes(int S, int m)
{
    const int nq = sub_quads(m);
    return (size_t)(S * nq + 1) * kSbGroup + (size_t)8 * (S % 8 != 0 ? kRing4Wave : kRingWave);
}

size_t jit_lds_bytes(int S, int m)
{
    const int nq = sub_quads(m);
    return (size_t)8 * nq * kSbGroup + (size_t)8 * (S % 8 != 0 ? kRing4Wave : kRingWave);
}

size_t lines_lds_bytes(int S, int m, int waves)
{
    return (size_t)(S * m + 1) * kI8ColBytes + (size_t)waves * kRingWave;
}

}  // namespace q4k

// q4k_device.h -- device helpers shared by the GEMV kernels (q4k_kernels.hip,
// q4k_mfma.hip, q4k_dpp.hip): the exact eight-weight dot of the f32-x
// kernels, the superblock header decode, loads, DPP moves and wave reductions.
// Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// --------------------------------------------------------------- helpers
// One weight from a code held as an fp16 subnormal in half H of p (the code
// q in the low mantissa bits: q 2^-24, or q 2^-20 for a high nibble masked
// in place), scaled by s = d sc 2^24 (or 2^20) and less mn = dmin m:
// fl32(d sc q - dmin m) with one rounding (the product is exact inside the
// fma), the weight the format defines.
template <int H>
__device__ __forceinline__ float weight_mix(uint32_t p, float s, float mn)
{
    const half2_t h = __builtin_bit_cast(half2_t, p);
    return __builtin_fmaf((float)(H ? h.y : h.x), s, -mn);
}

// Eight weights of one dword D (bytes 4u..4u+3 of a chunk: low nibbles in
// sub-block 2c, high nibbles in 2c+1) times their x, added in f64: each
// weight as weight_mix rounds it, each product exact in f64 (24-bit by
// 24-bit significands, no f32 range limit), so the sums' only error is f64
// rounding.  xl = x[4u], x[4u+2], x[4u+1], x[4u+3] (low nibbles); xh the same
// positions + 32 (high nibbles), as float4 or, converted ahead, as X4D.
// sl, sh: d sc_2c 2^24 and d sc_2c+1 2^20; ml, mh: dmin m of the two
// sub-blocks.
struct X4D {
    double x, y, z, w;
};

template <typename X4>
__device__ __forceinline__ void dot8_exact(uint32_t D, const X4& xl, const X4& xh, float sl,
                                           float sh, float ml, float mh, double& alo, double& ahi)
{
    const uint32_t p0 = D & 0x000F000Fu;   // bytes 0, 2 low nibble  = q * 2^-24
    const uint32_t p1 = D & 0x00F000F0u;   // bytes 0, 2 high nibble = q * 2^-20
    const uint32_t d8 = D >> 8;
    const uint32_t p2 = d8 & 0x000F000Fu;  // bytes 1, 3 low nibble
    const uint32_t p3 = d8 & 0x00F000F0u;  // bytes 1, 3 high nibble
    alo = __builtin_fma((double)weight_mix<0>(p0, sl, ml), (double)xl.x, alo);
    alo = __builtin_fma((double)weight_mix<1>(p0, sl, ml), (double)xl.y, alo);
    alo = __builtin_fma((double)weight_mix<0>(p2, sl, ml), (double)xl.z, alo);
    alo = __builtin_fma((double)weight_mix<1>(p2, sl, ml), (double)xl.w, alo);
    ahi = __builtin_fma((double)weight_mix<0>(p1, sh, mh), (double)xh.x, ahi);
    ahi = __builtin_fma((double)weight_mix<1>(p1, sh, mh), (double)xh.y, ahi);
    ahi = __builtin_fma((double)weight_mix<0>(p3, sh, mh), (double)xh.z, ahi);
    ahi = __builtin_fma((double)weight_mix<1>(p3, sh, mh), (double)xh.w, ahi);
}

// The factors of chunk c's weights for dot8_exact: sl = d sc_2c 2^24, sh =
// d sc_2c+1 2^20 (exact: an 11-bit d times a 6-bit sc, times a power of
// two), ml, mh = dmin m of the two sub-blocks (exact).
struct ChunkScales {
    float sl, sh, ml, mh;
};

// Header dwords: h.x = d | dmin << 16, h.y = s[0..3], h.z = s[4..7],
// h.w = s[8..11].  Chunk c needs sub-blocks j = 2c, 2c+1:
//   j < 4 : sc_j = s[j] & 63,                      m_j = s[j+4] & 63
//   j >= 4: sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4
//           m_j  = (s[j+4] >> 4) | (s[j]   >> 6) << 4
// Both forms take bytes 2(c&1), 2(c&1)+1 of their dwords, so one shift
// serves both; sh = 16 (c & 1) and sel = all ones for c < 2, else 0 (lane
// constants) pick the form without a branch.
__device__ __forceinline__ ChunkScales decode_header(const uint4& h, uint32_t shift, uint32_t sel)
{
    const half2_t dd = __builtin_bit_cast(half2_t, h.x);
    const float d = (float)dd.x;
    const float dmin = (float)dd.y;
    const uint32_t y = h.y >> shift;
    const uint32_t z = h.z >> shift;
    const uint32_t wv = h.w >> shift;
    const uint32_t sc_b = (wv & 0x0F0Fu) | ((y >> 2) & 0x3030u);
    const uint32_t m_b = ((wv >> 4) & 0x0F0Fu) | ((z >> 2) & 0x3030u);
    const uint32_t sc = ((y & 0x3F3Fu) & sel) | (sc_b & ~sel);
    const uint32_t mm = ((z & 0x3F3Fu) & sel) | (m_b & ~sel);
    ChunkScales s;
    s.sl = d * (float)(sc & 0xFFu) * 16777216.0f;
    s.sh = d * (float)((sc >> 8) & 0xFFu) * 1048576.0f;
    s.ml = dmin * (float)(mm & 0xFFu);
    s.mh = dmin * (float)((mm >> 8) & 0xFFu);
    return s;
}

// v of another lane of the wave, chosen by the DPP control CTRL (all rows
// and banks enabled)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        v += __shfl_xor(v, off, 64);
    }
    return v;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load16(const uint8_t* p)
{
    return *reinterpret_cast<const uint4*>(p);
}



}  // namespace q4k

// q4k_device.h -- device helpers shared by the GEMV kernels (q4k_kernels.hip,
// q4k_mfma.hip, q4k_dpp.hip): fp16 half access, the eight-code fma_mix dot,
// the superblock header decode, loads, DPP moves and wave reductions.
// Internal.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// --------------------------------------------------------------- helpers
__device__ __forceinline__ float fmix_lo(uint32_t p, float xv, float acc)
{
    const half2_t h = __builtin_bit_cast(half2_t, p);
    return __builtin_fmaf((float)h.x, xv, acc);
}

__device__ __forceinline__ float fmix_hi(uint32_t p, float xv, float acc)
{
    const half2_t h = __builtin_bit_cast(half2_t, p);
    return __builtin_fmaf((float)h.y, xv, acc);
}

// Eight codes of one dword D (bytes 4u..4u+3 of a chunk) against their x.
// xl = x[4u], x[4u+2], x[4u+1], x[4u+3]        (low nibbles, sub-block 2c)
// xh = the same positions + 32, divided by 16  (high nibbles, sub-block 2c+1)
__device__ __forceinline__ void dot8(uint32_t D, const float4& xl, const float4& xh,
                                     float& alo, float& ahi)
{
    const uint32_t p0 = D & 0x000F000Fu;   // bytes 0, 2 low nibble  = q * 2^-24
    const uint32_t p1 = D & 0x00F000F0u;   // bytes 0, 2 high nibble = q * 2^-20
    const uint32_t d8 = D >> 8;
    const uint32_t p2 = d8 & 0x000F000Fu;  // bytes 1, 3 low nibble
    const uint32_t p3 = d8 & 0x00F000F0u;  // bytes 1, 3 high nibble
    alo = fmix_lo(p0, xl.x, alo);
    alo = fmix_hi(p0, xl.y, alo);
    alo = fmix_lo(p2, xl.z, alo);
    alo = fmix_hi(p2, xl.w, alo);
    ahi = fmix_lo(p1, xh.x, ahi);
    ahi = fmix_hi(p1, xh.y, ahi);
    ahi = fmix_lo(p3, xh.z, ahi);
    ahi = fmix_hi(p3, xh.w, ahi);
}

struct ChunkScales {
    float d24;    // d * 2^24 (the fma_mix codes' values are q * 2^-24)
    float dmin;
    float sc_lo, sc_hi, m_lo, m_hi;
};

// Header dwords: h.x = d | dmin << 16, h.y = s[0..3], h.z = s[4..7],
// h.w = s[8..11].  Chunk c needs sub-blocks j = 2c, 2c+1:
//   j < 4 : sc_j = s[j] & 63,                      m_j = s[j+4] & 63
//   j >= 4: sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4
//           m_j  = (s[j+4] >> 4) | (s[j]   >> 6) << 4
// Both forms take bytes 2(c&1), 2(c&1)+1 of their dwords, so one shift
// serves both; the lane picks its form with a select.
__device__ __forceinline__ ChunkScales decode_header(const uint4& h, int c)
{
    ChunkScales s;
    const half2_t dd = __builtin_bit_cast(half2_t, h.x);
    s.d24 = (float)dd.x * 16777216.0f;
    s.dmin = (float)dd.y;
    const uint32_t sh = (uint32_t)(c & 1) * 16u;
    const uint32_t y = h.y >> sh;
    const uint32_t z = h.z >> sh;
    const uint32_t wv = h.w >> sh;
    const uint32_t sc_a = y & 0x3F3Fu;
    const uint32_t m_a = z & 0x3F3Fu;
    const uint32_t sc_b = (wv & 0x0F0Fu) | ((y >> 2) & 0x3030u);
    const uint32_t m_b = ((wv >> 4) & 0x0F0Fu) | ((z >> 2) & 0x3030u);
    const uint32_t sc = c < 2 ? sc_a : sc_b;
    const uint32_t mm = c < 2 ? m_a : m_b;
    s.sc_lo = (float)(sc & 0xFFu);
    s.sc_hi = (float)((sc >> 8) & 0xFFu);
    s.m_lo = (float)(mm & 0xFFu);
    s.m_hi = (float)((mm >> 8) & 0xFFu);
    return s;
}

// Scales of chunk g (sub-blocks 2g, 2g+1) of a header, d unscaled; sh =
// 16 (g & 1) and sel = all ones for g < 2, else 0 (lane constants).
struct ChunkScalesD {
    float d, dmin, sc_lo, sc_hi, m_lo, m_hi;
};

__device__ __forceinline__ ChunkScalesD decode_chunk(const uint4& h, uint32_t sh, uint32_t sel)
{
    ChunkScalesD s;
    const half2_t dd = __builtin_bit_cast(half2_t, h.x);
    s.d = (float)dd.x;
    s.dmin = (float)dd.y;
    const uint32_t y = h.y >> sh;
    const uint32_t z = h.z >> sh;
    const uint32_t wv = h.w >> sh;
    const uint32_t sc_b = (wv & 0x0F0Fu) | ((y >> 2) & 0x3030u);
    const uint32_t m_b = ((wv >> 4) & 0x0F0Fu) | ((z >> 2) & 0x3030u);
    const uint32_t sc = ((y & 0x3F3Fu) & sel) | (sc_b & ~sel);
    const uint32_t mm = ((z & 0x3F3Fu) & sel) | (m_b & ~sel);
    s.sc_lo = (float)(sc & 0xFFu);
    s.sc_hi = (float)((sc >> 8) & 0xFFu);
    s.m_lo = (float)(mm & 0xFFu);
    s.m_hi = (float)((mm >> 8) & 0xFFu);
    return s;
}

// v of another lane of the wave, chosen by the DPP control CTRL (all rows
// and banks enabled)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float wave_sum(float v)
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

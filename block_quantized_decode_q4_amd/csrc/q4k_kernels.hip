// q4k_kernels.hip -- HIP kernels for the Q4_K fused dequantize-and-multiply
// GEMV on CDNA4 (gfx950, wave64).  Launchers are in q4k_api.hip.
//
// Problem (see include/q4k.h for the page citations): y[b][r] =
// sum_c W[r][c] * x[b][c], W stored as GGUF Q4_K superblocks of 144 bytes /
// 256 weights, w = d*sc_j*q - dmin*m_j.
//
// Design (MI355X-first; the pages' CUDA kernels are prior art only):
//  * Lane map.  Four lanes share a superblock; lane t owns the 64-element
//    chunk c = t % 4 of superblock t / 4, i.e. 32 quant bytes (two 16-byte
//    loads) and the two sub-blocks 2c (low nibbles) and 2c+1 (high
//    nibbles).  One wave pass covers 16 superblocks = 4096 elements (a
//    "span").  Per superblock and row each lane issues three dwordx4 loads:
//    the 16-byte header (d, dmin, scales) and its 32 quant bytes.
//  * Nibble decode without conversions.  A 4-bit code placed in the low
//    mantissa bits of an fp16 is the subnormal q*2^-24 (or q*2^-20 for a
//    high nibble masked in place), exactly.  One AND turns a dword of
//    codes into two such fp16 values, and v_fma_mix_f32 multiplies an fp16
//    half of a register by an f32 x and accumulates in f32.  Eight weights
//    cost 5 integer ops + 8 fma_mix.  The 2^-24 is folded into d, and the
//    high-nibble 16 into x (x of high-nibble elements is staged as x/16, an
//    exact power-of-two scaling).
//  * Scales factored out.  Per lane and superblock:
//      acc += d*2^24 * (sc_lo*A_lo + sc_hi*A_hi) - dmin*(m_lo*X_lo + m_hi*X_hi)
//    with A = sum q*x over the lane's 32 elements of each sub-block and X =
//    sum x over the same elements.  X depends only on x, so the x stager
//    computes it once per workgroup: the min term costs nothing per weight.
//  * x stager (LDS).  A workgroup stages x (or a K-chunk of it) into LDS in
//    lane order -- [vector][span][v = 0..15][lane] float4 -- so every
//    ds_read_b128 of a wave reads 1 KiB of consecutive LDS (no bank
//    conflicts), plus X per lane.  With one span and one vector, x is then
//    held in 64 VGPRs per lane for the whole row loop.
//  * K-chunked path.  When x does not fit the single-stage LDS budget, it is
//    staged spans_per_chunk spans at a time; each lane's partial sums are
//    parked in LDS between chunks, so the accumulation order -- and the
//    result -- is identical to the single-stage path.
//  * Multi-output scheduling.  A workgroup owns rows_per_block consecutive
//    rows; its waves take groups of R rows round-robin and decode R rows per
//    pass against one read of x, and the row loop streams each row once.
//  * Per-row reduction: 64 lane partials -> one value with a butterfly of
//    cross-lane adds; y is written once per row (overwrite).
//  * m-batched (m <= 8): each decoded code feeds m accumulators.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_kernels.h"

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
    float d24;    // d * 2^24
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

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        v += __shfl_xor(v, off, 64);
    }
    return v;
}

__device__ __forceinline__ uint4 load16(const uint8_t* p)
{
    return *reinterpret_cast<const uint4*>(p);
}

// ------------------------------------------------------------ x stager
// Stage spans [span0, span0 + nsp) of every vector into LDS in lane order
// and compute the per-lane sums X.  Slot ((b*nsp + sp)*16 + v)*64 + lane
// holds, for superblock sb = (span0+sp)*16 + lane/4, chunk c = lane%4,
// u = v/2, h = v%2: x[b][sb*256 + 64c + 32h + 4u + {0,2,1,3}] (times 1/16
// when h = 1).  Superblocks past the row end stage zeros.
template <int M>
__device__ __forceinline__ void stage_x(const float* __restrict__ x, int k, int S, int span0,
                                        int nsp, float4* xs, float2* sums, int tid, int nthreads)
{
    const int per_vec = nsp * 1024;
    for (int slot = tid; slot < M * per_vec; slot += nthreads) {
        const int b = slot / per_vec;
        const int rem = slot - b * per_vec;
        const int sp = rem >> 10;
        const int v = (rem >> 6) & 15;
        const int ln = rem & 63;
        const int sb = (span0 + sp) * 16 + (ln >> 2);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (sb < S) {
            const int c = ln & 3;
            const int u = v >> 1;
            const int h = v & 1;
            const int e = sb * 256 + 64 * c + 32 * h + 4 * u;
            const float4 g = *reinterpret_cast<const float4*>(x + (size_t)b * k + e);
            const float sc = h ? 0.0625f : 1.0f;
            o = make_float4(g.x * sc, g.z * sc, g.y * sc, g.w * sc);
        }
        xs[slot] = o;
    }
    __syncthreads();
    for (int t = tid; t < M * nsp * 64; t += nthreads) {
        const int bsp = t >> 6;
        const int ln = t & 63;
        const float4* base = xs + bsp * 1024 + ln;
        float lo = 0.f, hi = 0.f;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float4 a = base[(2 * u) * 64];
            const float4 q = base[(2 * u + 1) * 64];
            lo += (a.x + a.y) + (a.z + a.w);
            hi += (q.x + q.y) + (q.z + q.w);
        }
        sums[t] = make_float2(lo, hi * 16.0f);   // undo the exact 1/16 scaling
    }
    __syncthreads();
}

// ---------------------------------------------------------------- GEMV
template <int M, int R, int NW, bool XREG>
__global__ void __launch_bounds__(NW * 64)
gemv_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x, float* __restrict__ y,
            int n, int k, int S, int rows_per_block, int spans_per_chunk)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = lane & 3;
    const int sbl = lane >> 2;

    const int nspans = (S + 15) >> 4;
    const int chunk_spans = spans_per_chunk < nspans ? spans_per_chunk : nspans;
    const int nchunks = (nspans + chunk_spans - 1) / chunk_spans;
    float4* xs = reinterpret_cast<float4*>(smem);
    float2* sums = reinterpret_cast<float2*>(xs + M * chunk_spans * 1024);
    float* partial = reinterpret_cast<float*>(sums + M * chunk_spans * 64);

    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ngroups = (rows_here + R - 1) / R;
    const size_t row_bytes = (size_t)S * 144;

    for (int ch = 0; ch < nchunks; ++ch) {
        const int span0 = ch * chunk_spans;
        const int nsp = min(chunk_spans, nspans - span0);
        if (ch > 0) {
            __syncthreads();            // every wave is done with the previous chunk
        }
        stage_x<M>(x, k, S, span0, nsp, xs, sums, tid, NW * 64);

        float4 xr[XREG ? 16 : 1];
        float2 Xr = make_float2(0.f, 0.f);
        if constexpr (XREG) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                xr[v] = xs[v * 64 + lane];
            }
            Xr = sums[lane];
        }

        for (int g = wave; g < ngroups; g += NW) {
            float acc[R][M];
#pragma unroll
            for (int i = 0; i < R; ++i) {
#pragma unroll
                for (int b = 0; b < M; ++b) {
                    acc[i][b] = ch == 0 ? 0.f : partial[((g * R + i) * M + b) * 64 + lane];
                }
            }
            for (int sp = 0; sp < nsp; ++sp) {
                const int sb = (span0 + sp) * 16 + sbl;
                const bool sb_ok = sb < S;
                uint4 hd[R], qa[R], qb[R];
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const int rl = g * R + i;
                    if (sb_ok && rl < rows_here) {
                        const uint8_t* p = w + (size_t)(row0 + rl) * row_bytes + (size_t)sb * 144;
                        hd[i] = load16(p);
                        qa[i] = load16(p + 16 + 32 * c);
                        qb[i] = load16(p + 32 + 32 * c);
                    } else {
                        hd[i] = make_uint4(0u, 0u, 0u, 0u);
                        qa[i] = make_uint4(0u, 0u, 0u, 0u);
                        qb[i] = make_uint4(0u, 0u, 0u, 0u);
                    }
                }
                float alo[R][M], ahi[R][M];
#pragma unroll
                for (int i = 0; i < R; ++i) {
#pragma unroll
                    for (int b = 0; b < M; ++b) {
                        alo[i][b] = 0.f;
                        ahi[i][b] = 0.f;
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    float4 xl[M], xh[M];
                    if constexpr (XREG) {
                        xl[0] = xr[2 * u];
                        xh[0] = xr[2 * u + 1];
                    } else {
#pragma unroll
                        for (int b = 0; b < M; ++b) {
                            const float4* xb = xs + (b * nsp + sp) * 1024 + lane;
                            xl[b] = xb[(2 * u) * 64];
                            xh[b] = xb[(2 * u + 1) * 64];
                        }
                    }
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        const uint4& q4 = u < 4 ? qa[i] : qb[i];
                        const int uu = u & 3;
                        const uint32_t D = uu == 0 ? q4.x : uu == 1 ? q4.y : uu == 2 ? q4.z : q4.w;
#pragma unroll
                        for (int b = 0; b < M; ++b) {
                            dot8(D, xl[b], xh[b], alo[i][b], ahi[i][b]);
                        }
                    }
                }
                float2 X[M];
                if constexpr (XREG) {
                    X[0] = Xr;
                } else {
#pragma unroll
                    for (int b = 0; b < M; ++b) {
                        X[b] = sums[(b * nsp + sp) * 64 + lane];
                    }
                }
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    const ChunkScales s = decode_header(hd[i], c);
#pragma unroll
                    for (int b = 0; b < M; ++b) {
                        float t1 = s.sc_lo * alo[i][b];
                        t1 = __builtin_fmaf(s.sc_hi, ahi[i][b], t1);
                        float t2 = s.m_lo * X[b].x;
                        t2 = __builtin_fmaf(s.m_hi, X[b].y, t2);
                        acc[i][b] = __builtin_fmaf(s.d24, t1, acc[i][b]);
                        acc[i][b] = __builtin_fmaf(-s.dmin, t2, acc[i][b]);
                    }
                }
            }
            if (ch == nchunks - 1) {
#pragma unroll
                for (int i = 0; i < R; ++i) {
#pragma unroll
                    for (int b = 0; b < M; ++b) {
                        const float v = wave_sum(acc[i][b]);
                        const int rl = g * R + i;
                        if (lane == 0 && rl < rows_here) {
                            y[(size_t)b * n + row0 + rl] = v;
                        }
                    }
                }
            } else {
#pragma unroll
                for (int i = 0; i < R; ++i) {
#pragma unroll
                    for (int b = 0; b < M; ++b) {
                        partial[((g * R + i) * M + b) * 64 + lane] = acc[i][b];
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------- dequant
// One thread per (superblock, chunk c, dword u): decodes 8 weights and
// writes them as two float4.  w = fma(d*sc, q, -dmin*m); d*sc and dmin*m
// are exact in f32 and so is d*sc*q, so the fma's single rounding is the
// rounding of the exact value.
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t* __restrict__ w, float* __restrict__ out, int64_t nsb)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t sb = t >> 5;
    if (sb >= nsb) {
        return;
    }
    const int part = (int)(t & 31);
    const int c = part >> 3;
    const int u = part & 7;
    const uint8_t* p = w + sb * 144;
    const uint4 h = load16(p);
    const uint32_t D = *reinterpret_cast<const uint32_t*>(p + 16 + 32 * c + 4 * u);
    const half2_t dd = __builtin_bit_cast(half2_t, h.x);
    const float d = (float)dd.x;
    const float dmin = (float)dd.y;
    const uint32_t sh = (uint32_t)(c & 1) * 16u;
    const uint32_t y = h.y >> sh;
    const uint32_t z = h.z >> sh;
    const uint32_t wv = h.w >> sh;
    const uint32_t sc = c < 2 ? (y & 0x3F3Fu) : ((wv & 0x0F0Fu) | ((y >> 2) & 0x3030u));
    const uint32_t mm = c < 2 ? (z & 0x3F3Fu) : (((wv >> 4) & 0x0F0Fu) | ((z >> 2) & 0x3030u));
    const float dsc_lo = d * (float)(sc & 0xFFu);
    const float dsc_hi = d * (float)((sc >> 8) & 0xFFu);
    const float dm_lo = dmin * (float)(mm & 0xFFu);
    const float dm_hi = dmin * (float)((mm >> 8) & 0xFFu);
    float4 lo, hi;
    lo.x = __builtin_fmaf(dsc_lo, (float)(D & 15u), -dm_lo);
    lo.y = __builtin_fmaf(dsc_lo, (float)((D >> 8) & 15u), -dm_lo);
    lo.z = __builtin_fmaf(dsc_lo, (float)((D >> 16) & 15u), -dm_lo);
    lo.w = __builtin_fmaf(dsc_lo, (float)((D >> 24) & 15u), -dm_lo);
    hi.x = __builtin_fmaf(dsc_hi, (float)((D >> 4) & 15u), -dm_hi);
    hi.y = __builtin_fmaf(dsc_hi, (float)((D >> 12) & 15u), -dm_hi);
    hi.z = __builtin_fmaf(dsc_hi, (float)((D >> 20) & 15u), -dm_hi);
    hi.w = __builtin_fmaf(dsc_hi, (float)(D >> 28), -dm_hi);
    float* o = out + sb * 256 + 64 * c + 4 * u;
    *reinterpret_cast<float4*>(o) = lo;
    *reinterpret_cast<float4*>(o + 32) = hi;
}

// --------------------------------------------------------- calibration
// Streaming read of n16 16-byte words with the same load width the GEMV
// uses; the xor checksum keeps the loads alive.
__global__ void __launch_bounds__(256)
read_kernel(const uint4* __restrict__ buf, size_t n16, float* __restrict__ out)
{
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = buf[i];
        const uint4 b = buf[i + stride];
        const uint4 c = buf[i + 2 * stride];
        const uint4 d = buf[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
        acc ^= c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = buf[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
    }
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0) {
        part[threadIdx.x >> 6] = acc;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        out[blockIdx.x] = (float)((part[0] ^ part[1] ^ part[2] ^ part[3]) & 0xFFFFu);
    }
}

// -------------------------------------------------------------- launch
template <int M, int R, int NW, bool XREG>
static hipError_t launch_one(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                             hipStream_t stream)
{
    hipLaunchKernelGGL((gemv_kernel<M, R, NW, XREG>), dim3(p.grid), dim3(NW * 64), p.lds_bytes,
                       stream, w, x, y, p.n, p.k, p.S, p.rows_per_block, p.spans_per_chunk);
    return hipGetLastError();
}

template <int M>
static hipError_t launch_m(const GemvPlan& p, const uint8_t* w, const float* x, float* y,
                           hipStream_t stream)
{
    if constexpr (M == 1) {
        if (p.x_in_registers) {
            if (p.waves_per_block == 8) {
                if (p.rows_per_wave == 4) return launch_one<1, 4, 8, true>(p, w, x, y, stream);
                if (p.rows_per_wave == 2) return launch_one<1, 2, 8, true>(p, w, x, y, stream);
                return launch_one<1, 1, 8, true>(p, w, x, y, stream);
            }
            if (p.rows_per_wave == 4) return launch_one<1, 4, 4, true>(p, w, x, y, stream);
            if (p.rows_per_wave == 2) return launch_one<1, 2, 4, true>(p, w, x, y, stream);
            return launch_one<1, 1, 4, true>(p, w, x, y, stream);
        }
        if (p.waves_per_block == 8) {
            if (p.rows_per_wave == 4) return launch_one<1, 4, 8, false>(p, w, x, y, stream);
            if (p.rows_per_wave == 2) return launch_one<1, 2, 8, false>(p, w, x, y, stream);
            return launch_one<1, 1, 8, false>(p, w, x, y, stream);
        }
        if (p.rows_per_wave == 4) return launch_one<1, 4, 4, false>(p, w, x, y, stream);
        if (p.rows_per_wave == 2) return launch_one<1, 2, 4, false>(p, w, x, y, stream);
        return launch_one<1, 1, 4, false>(p, w, x, y, stream);
    } else {
        if (p.waves_per_block == 8) {
            if (p.rows_per_wave == 2) return launch_one<M, 2, 8, false>(p, w, x, y, stream);
            return launch_one<M, 1, 8, false>(p, w, x, y, stream);
        }
        if (p.rows_per_wave == 2) return launch_one<M, 2, 4, false>(p, w, x, y, stream);
        return launch_one<M, 1, 4, false>(p, w, x, y, stream);
    }
}

hipError_t launch_gemv(const GemvPlan& p, const void* w, const float* x, float* y,
                       hipStream_t stream)
{
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    switch (p.m) {
    case 1: return launch_m<1>(p, wb, x, y, stream);
    case 2: return launch_m<2>(p, wb, x, y, stream);
    case 3: return launch_m<3>(p, wb, x, y, stream);
    case 4: return launch_m<4>(p, wb, x, y, stream);
    case 5: return launch_m<5>(p, wb, x, y, stream);
    case 6: return launch_m<6>(p, wb, x, y, stream);
    case 7: return launch_m<7>(p, wb, x, y, stream);
    case 8: return launch_m<8>(p, wb, x, y, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dequant(const void* w, float* out, int64_t nsb, hipStream_t stream)
{
    const int64_t threads = nsb * 32;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(w), out, nsb);
    return hipGetLastError();
}

hipError_t launch_read(const void* buf, size_t n16, float* out, hipStream_t stream)
{
    hipLaunchKernelGGL(read_kernel, dim3(kReadBlocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(buf), n16, out);
    return hipGetLastError();
}

}  // namespace q4k

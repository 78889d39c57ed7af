// q4k_xrep.h -- the integer representation of x used by the line-streamed
// integer kernels (q4k_dpp.hip: vector ALU; q4k_mfma.hip: matrix cores).
// Internal.
//
// Per 32-element sub-block of one vector (the unit that shares d*sc_j and
// dmin*m_j in the Q4_K format):
//  * mx = the largest |x| (NaN left out), sigma = 30 - E for mx = f * 2^E
//    with f in [1/2, 1), so that mx * 2^sigma lies in [2^29, 2^30) (sigma =
//    0 when mx = 0, 30 when mx is infinite: frexp gives it exponent 0).
//    sigma spans -98 .. 178, so the scale 2^-sigma is kept in f64 and no
//    range is clamped;
//  * v = x * 2^sigma (exact for every element that does not round to
//    zero), xi = rint(v) with |xi| < 2^30, written as four signed base-256
//    digits (the bytes of xi + 0x80808080, each minus 128), so that int8
//    products of the 4-bit codes with the digits sum exactly in int32;
//  * an element is certified when x = 0 or 2^16 <= |v| <= 2^30: then xi
//    carries it to a relative error of 2^-17 at most.  An uncertified
//    element (a value below 2^-13 of its sub-block's largest, or inf/NaN)
//    is left out of the digits (xi := 0) and out of XI; the
//    kernels add its weight times its exact x separately: from a short list
//    of the column's first kCorr such elements, kept beside the digits,
//    and, for a column with more, from x in global memory, where the same
//    test picks them out again.
// With a relative error of 2^-17 per certified element, an output's error
// from x is at most 2^-17 sum |w||x| whatever the weights; the digit sums
// are exact and are scaled with one rounding per sub-block (subblock_term),
// so the 1e-5 sum |w||x| bound holds for every input, and non-finite x
// propagate as IEEE arithmetic does.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

constexpr float kCertRel = 0x1p-17f;
constexpr int kCorr = 4;             // exact corrections listed per column

// grid exponent of a sub-block from its largest finite |x|
__device__ __forceinline__ int grid_sigma(float mx)
{
    return mx > 0.f ? 30 - __builtin_amdgcn_frexp_expf(mx) : 0;
}

// 2^-sigma as f64 (sigma in -98 .. 178: a normal double), and back
__device__ __forceinline__ double grid_scale(int sigma)
{
    return __builtin_bit_cast(double, (uint64_t)(1023 - sigma) << 52);
}

__device__ __forceinline__ int grid_sigma_of(double s)
{
    return 1023 - (int)((__builtin_bit_cast(uint64_t, s) >> 52) & 0x7FFu);
}

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

// One element on the grid: u = xi + 0x80808080 (its bytes are the digits
// plus 128), and whether the element is certified (1) or not (0): x = 0,
// or 2^16 <= |x 2^sigma| <= 2^30, where the rounding to an integer errs by
// at most 1/2 <= 2^-17 |x 2^sigma|.  Everything else -- values below 2^-13
// of the sub-block's largest, inf and NaN (whose v is not finite or not a
// number) -- is uncertified and leaves the digits (xi = 0).  Branch-free:
// the callers exchange results between lanes, which needs every lane active.
__device__ __forceinline__ void grid_element(float x, int sigma, uint32_t& u, int& cert)
{
    const float v = __builtin_amdgcn_ldexpf(x, sigma);
    const float a = fabsf(v);
    cert = ((a >= 65536.f) & (a <= 0x1p30f)) | (x == 0.f);
    const int xi = cert ? (int)__builtin_rintf(v) : 0;
    u = (uint32_t)xi + 0x80808080u;
}

// Four elements' u -> four digit planes: plane l holds digit l of elements
// 0..3 in bytes 0..3, as signed bytes.
__device__ __forceinline__ void digit_planes(const uint32_t (&u)[4], uint32_t (&d)[4])
{
    const uint32_t lo01 = __builtin_amdgcn_perm(u[1], u[0], 0x05010400u);   // b0 b0 b1 b1
    const uint32_t lo23 = __builtin_amdgcn_perm(u[3], u[2], 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(u[1], u[0], 0x07030602u);   // b2 b2 b3 b3
    const uint32_t hi23 = __builtin_amdgcn_perm(u[3], u[2], 0x07030602u);
    d[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u) ^ 0x80808080u;
    d[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u) ^ 0x80808080u;
    d[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u) ^ 0x80808080u;
    d[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u) ^ 0x80808080u;
}

// T = t0 + 256 t1 + 65536 t2 + 2^24 t3 from four exact digit sums, exactly
// (|t_l| < 2^19 each, so the pairs fit int32 and T fits f64)
__device__ __forceinline__ double digits_exact(int t0, int t1, int t2, int t3)
{
    const int p = t0 + (t1 << 8);
    const int q = t2 + (t3 << 8);
    return __builtin_fma((double)q, 65536.0, (double)p);
}

// Exclusive prefix sum and total of v over the 16 lanes of a DPP row
// (every lane of the wave active): a Hillis-Steele scan by row_shr (lanes
// shifted in from outside the row read 0), the total by row_share:15.
__device__ __forceinline__ int row16_scan(int v, int& total)
{
    int incl = v;
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);   // row_shr:1
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);   // row_shr:2
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);   // row_shr:4
    incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);   // row_shr:8
    total = __builtin_amdgcn_update_dpp(0, incl, 0x15F, 0xF, 0xF, false);  // row_share:15
    return incl - v;
}

// The grid conversion of the 16 consecutive elements a lane holds (half a
// sub-block; lanes 2p and 2p + 1 hold one sub-block and meet through DPP,
// the 16 lanes of a row hold one 256-element column and meet through a row
// scan).  Every lane of the wave must call it (DPP, row scan).
struct Conv16 {
    uint32_t plane[4][4];   // plane[l][t]: digit l of elements 4t .. 4t+3, signed bytes
    double xsum;            // XI of the lane's sub-block (certified elements)
    double xsum16;          // XI of the lane's own 16 elements
    int sigma;              // the sub-block's grid exponent
    uint32_t uncmask;       // bit i: element i is uncertified
    int first;              // its index among the column's uncertified elements
    int total;              // uncertified elements of the column
};

__device__ __forceinline__ Conv16 convert16(const float (&e)[16])
{
    Conv16 c;
    // largest |x| (NaN left out by the IEEE max; an infinity makes mx
    // infinite, whose frexp exponent is 0: sigma = 30, a grid that still
    // carries every element it certifies, the sub-block's other large
    // values going to the exact terms)
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        mx = fmaxf(mx, fabsf(e[i]));
    }
    mx = fmaxf(mx, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                       0, __builtin_bit_cast(int, mx), 0xB1, 0xF, 0xF, false)));   // lane ^ 1
    c.sigma = grid_sigma(mx);
    c.uncmask = 0;
    int ps[4] = {0, 0, 0, 0};                   // digit-plane sums of the lane's elements
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        uint32_t u[4], d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int cert;
            grid_element(e[4 * t + i], c.sigma, u[i], cert);
            c.uncmask |= cert ? 0u : 1u << (4 * t + i);
        }
        digit_planes(u, d);
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            c.plane[l][t] = d[l];
            ps[l] = __builtin_amdgcn_sdot4((int)d[l], 0x01010101, ps[l], false);
        }
    }
    c.xsum16 = digits_exact(ps[0], ps[1], ps[2], ps[3]);
    // the sub-block's plane sums (pair by DPP), |sum| <= 32 * 128: XI exactly
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        ps[l] += __builtin_amdgcn_update_dpp(0, ps[l], 0xB1, 0xF, 0xF, false);
    }
    c.xsum = digits_exact(ps[0], ps[1], ps[2], ps[3]);
    c.first = row16_scan(__builtin_popcount(c.uncmask), c.total);
    return c;
}

// One entry of a column's correction list: element index and exact x.
struct Corr {
    uint32_t e;
    float x;
};

// Write the lane's uncertified elements (e0: index of its first element in
// the column) into the column's list at their places in element order,
// while the list has room.
__device__ __forceinline__ void store_corrections(unsigned char* list, const Conv16& c,
                                                  const float (&e)[16], int e0)
{
    uint32_t m = c.uncmask;
    int idx = c.first;
    while (m != 0u && idx < kCorr) {
        const int i = __builtin_ctz(m);
        m &= m - 1u;
        // element i by masks (an indexed read would go through scratch memory)
        uint32_t xb = 0;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            xb |= __builtin_bit_cast(uint32_t, e[t]) & (0u - (uint32_t)(i == t));
        }
        Corr r;
        r.e = (uint32_t)(e0 + i);
        r.x = __builtin_bit_cast(float, xb);
        *reinterpret_cast<Corr*>(list + idx * 8) = r;
        ++idx;
    }
}


// One sub-block's term 2^-sigma * (D T - M XI) of a row, added to acc.  D
// and M are d*sc_j and dmin*m_j (exact f32), T = sum q xi and XI = sum xi
// (exact integers in f64).  M*XI is exact (17 + 35 bits), so the fma rounds
// D T - M XI once, at its own size: no cancellation between the two
// products (weights d sc q close to dmin m) loses what the weights' own
// magnitudes carry; the scaling by 2^-sigma is exact.
__device__ __forceinline__ double subblock_term(double acc, float Df, double T, float Mf,
                                                double XI, double s)
{
    const double p2 = (double)Mf * XI;
    const double r = __builtin_fma((double)Df, T, -p2);
    return __builtin_fma(r, s, acc);
}

// Code dword u (0..7, wave-uniform) of the lane's chunk, by masks rather
// than an indexed read (which the compiler would serve from scratch memory).
__device__ __forceinline__ uint32_t pick_code(const uint32_t (&D)[8], int u)
{
    uint32_t r = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        r |= D[t] & (0u - (uint32_t)(u == t));
    }
    return r;
}

// The exact terms of a column's uncertified elements for a lane holding
// chunk g of one row (codes D, scales d sc and dmin m of its two
// sub-blocks): fl32(d sc q - dmin m) * x in f64, the oracle's own
// arithmetic.  Up to kCorr of them come from the column's list (the lanes
// of the element's chunk add it); a column with more is scanned again from x
// in global memory (xg: the column's 256 values), each element tested as
// the conversion tested it (slo, shi: the grid scales of the lane's two
// sub-blocks).
__device__ __forceinline__ double column_corrections(double acc, uint32_t cnt,
                                                     const unsigned char* list,
                                                     const uint32_t (&D)[8], int g,
                                                     float Dlo, float Dhi, float Mlo, float Mhi,
                                                     double slo, double shi,
                                                     const float* __restrict__ xg)
{
    if (cnt <= (uint32_t)kCorr) {
        for (uint32_t k = 0; k < cnt; ++k) {
            const Corr c = *reinterpret_cast<const Corr*>(list + k * 8);
            const int e = __builtin_amdgcn_readfirstlane((int)c.e);
            const float xv = __builtin_bit_cast(
                float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, c.x)));
            const int hh = (e >> 5) & 1;
            const int b = e & 31;                           // code byte of the chunk
            const uint32_t q = (pick_code(D, b >> 2) >> (8 * (b & 3) + 4 * hh)) & 15u;
            const float wv = __builtin_fmaf(hh ? Dhi : Dlo, (float)q, -(hh ? Mhi : Mlo));
            const double t = (double)wv * (double)xv;       // exact
            acc = g == (e >> 6) ? acc + t : acc;
        }
        return acc;
    }
#pragma nounroll
    for (int hh = 0; hh < 2; ++hh) {
        const float4* src = reinterpret_cast<const float4*>(xg + 64 * g + 32 * hh);
        float4 xv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            xv[t] = src[t];
        }
        const int sigma = grid_sigma_of(hh ? shi : slo);
        const float Dw = hh ? Dhi : Dlo;
        const float Mw = hh ? Mhi : Mlo;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float xe[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t u;
                int cert;
                grid_element(xe[i], sigma, u, cert);
                const uint32_t q = (D[t] >> (8 * i + 4 * hh)) & 15u;
                const float wv = __builtin_fmaf(Dw, (float)q, -Mw);
                const double tv = (double)wv * (double)xe[i];
                acc = cert ? acc : acc + tv;
            }
        }
    }
    return acc;
}

}  // namespace q4k

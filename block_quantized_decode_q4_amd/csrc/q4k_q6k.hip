// q4k_q6k.hip -- the GEMV over Q6_K weights, y = W x for one vector: the
// other block format of the decode loop (realizar 0.8.5,
// q4k_gemv_cached.rs, `q6k_gemv_cached_async`: the same GEMV for an LM head
// stored as Q6_K; memra-engine 0.83.1, src/f16_ffi.rs,
// `memra_q6_K_dequant_f16`: 210-byte superblocks of 256 weights).
//
// Format (the GGUF Q6_K layout): ql[128] low four bits, qh[64] high two
// bits, sixteen int8 scales (scale s for elements 16 s .. 16 s + 15), fp16 d
// at byte 208.  Element e = 128 h + 32 t + l: low bits in ql byte
// 64 h + 32 (t % 2) + l (low nibble for t < 2, high for t >= 2), high bits
// in bits 2 t, 2 t + 1 of qh byte 32 h + l; w = d sc (q - 32), an exact
// product in f32 (at most 11 + 7 + 5 significant bits).
//
// Arithmetic (the integer representation of q4k_xrep.h): x on the
// per-32-element grid as four signed int8 digits; for each 16-element
// group (one scale) the codes q (0..63, positive int8 operands) against the
// digits give exact int32 sums T_l, T = sum q xi exactly in f64, and the
// group adds 2^-s d sc (T - 32 XI) (XI = sum xi of the group) to an f64 sum
// with one rounding (subblock_term).  Uncertified elements (far below their
// block's largest, inf, NaN) are added exactly as the oracle does.  Error
// at most 2^-17 sum |w||x| plus f64 rounding: within 1e-5 sum |w||x| for
// every input.
//
// Lane layout of a step (one superblock column of a 16-row tile): lane
// l = 16 Q + j takes row j and quadrant Q = 2 h + a of the superblock: the
// 64 elements 128 h + 32 t + 16 a + i (t < 4, i < 16), i.e. ql bytes
// 64 h + 16 a + i and 64 h + 32 + 16 a + i and qh bytes 128 + 32 h + 16 a + i
// and the four scales 8 h + 2 t + a.  The 16 lanes of a DPP row share one
// quadrant; lane j of it holds the digits of elements (t, 4 u .. 4 u + 3)
// for j = 4 t + u, broadcast to the row by row_newbcast folded into the dot
// instruction (as in q4k_dpp.hip).
//
// Stream: rows start on 16-byte boundaries (row_stride % 16 == 0), and a
// superblock column sits 210 c bytes into its row.  Each wave streams its
// tile's 16 rows in batches of BB bytes per row into a 512-byte ring per
// row in LDS, 512 bytes per row in flight in registers.  A load instruction
// reads 16 rows x 64 bytes, or, with w 128-byte aligned, 8 rows x one whole
// 128-byte line: a row's batches then start on the line holding its first
// byte, the row's bytes `phase` (a multiple of 16, below 128) into them.
// Where no row has a phase (64-byte pieces, or a row stride that is a
// multiple of 128) a batch is 256 bytes (two lines of a row back to back),
// else 128.  After each batch the wave computes the columns whose 210 bytes
// are in the ring for every row.  A field of a column starts 210 c mod 4 = 0
// or 2 bytes into a dword (the same for every row): the lanes read five
// aligned dwords and shift them by that wave-uniform amount.  The ring
// repeats its first 32 bytes after its end, so no field read wraps.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q4k_device.h"
#include "q4k_kernels.h"
#include "q4k_lines.h"
#include "q4k_xrep.h"

namespace q4k {

constexpr int kQ6Digits = 0;                             // four quadrants x sixteen 16-byte slots
constexpr int kQ6Sum = 4 * 16 * 16;                      // XI of each group, f64 [quadrant][t]
constexpr int kQ6Scale = kQ6Sum + 16 * 8;                // 2^-sigma, f64 [h][t]
constexpr int kQ6Word = kQ6Scale + 8 * 8;                // uncertified elements of the column
constexpr int kQ6List = kQ6Word + 16;                    // the first kCorr of them
constexpr int kQ6Col = kQ6List + kCorr * 8;
constexpr int kQ6Ring = 512;                             // ring bytes per row
constexpr int kQ6Row = kQ6Ring + 48;                     // + the 32-byte repeat, padded
constexpr int kQ6Wave = 16 * kQ6Row;

static_assert(kQ6Col % 16 == 0 && kQ6Row % 16 == 0, "LDS layout alignment");

// One v_dot4c_i32_i8 whose first operand is lane N of the DPP row.
#define Q6K_DOTB(ACC, X, C, N) \
    "v_dot4c_i32_i8_dpp %" #ACC ", %" #X ", %" #C " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n"
// Code dword u of groups t0 and t1 against the four digits of lanes
// N0 = 4 t0 + u and N1 = 4 t1 + u: accumulators 0-3 and 4-7.
#define Q6K_DOTU(C0, C1, N0, N1)                                              \
    Q6K_DOTB(0, 8, C0, N0) Q6K_DOTB(1, 9, C0, N0) Q6K_DOTB(2, 10, C0, N0)     \
    Q6K_DOTB(3, 11, C0, N0) Q6K_DOTB(4, 8, C1, N1) Q6K_DOTB(5, 9, C1, N1)     \
    Q6K_DOTB(6, 10, C1, N1) Q6K_DOTB(7, 11, C1, N1)
#define Q6K_OPERANDS                                                                          \
    : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]),     \
      "+v"(t[7])                                                                              \
    : "v"(xd.x), "v"(xd.y), "v"(xd.z), "v"(xd.w), "v"(c0[0]), "v"(c0[1]), "v"(c0[2]),         \
      "v"(c0[3]), "v"(c1[0]), "v"(c1[1]), "v"(c1[2]), "v"(c1[3])

// Digit sums of groups 2P and 2P + 1: t[0..3] += codes c0 (group 2P) against
// the digits of lanes 8P + u, t[4..7] += c1 (group 2P + 1) against lanes
// 8P + 4 + u.  Hazards as in q4k_dpp.hip's dot_step: five wait states before
// (a DPP operand after a VALU or EXEC write), three after (a dot result read
// by the next VALU instruction), each accumulator rewritten eight
// instructions after its last write.
template <int P>
__device__ __forceinline__ void q6_dot_pair(const uint4& xd, const int (&c0)[4], const int (&c1)[4],
                                            int (&t)[8])
{
    if constexpr (P == 0) {
        asm("s_nop 4\n"
            Q6K_DOTU(12, 16, 0, 4) Q6K_DOTU(13, 17, 1, 5) Q6K_DOTU(14, 18, 2, 6)
            Q6K_DOTU(15, 19, 3, 7)
            "s_nop 2\n" Q6K_OPERANDS);
    } else {
        asm("s_nop 4\n"
            Q6K_DOTU(12, 16, 8, 12) Q6K_DOTU(13, 17, 9, 13) Q6K_DOTU(14, 18, 10, 14)
            Q6K_DOTU(15, 19, 11, 15)
            "s_nop 2\n" Q6K_OPERANDS);
    }
}

#undef Q6K_OPERANDS
#undef Q6K_DOTU
#undef Q6K_DOTB

// Convert 16 consecutive x values (group G of 16: column G / 16, elements
// 16 (G % 16) ..) into the column's slots: 16 g = 128 h + 32 t + 16 a gives
// quadrant 2 h + a, slots 4 t .. 4 t + 3; the group's XI; the 32-element
// block's grid scale; the column's uncertified elements.  Every lane of the
// wave calls this (DPP, row scan); `store` is false past the last column.
__device__ __forceinline__ void convert_group_q6(const float4 (&v)[4], int G, bool store,
                                                 unsigned char* xs)
{
    const float e[16] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w,
                         v[2].x, v[2].y, v[2].z, v[2].w, v[3].x, v[3].y, v[3].z, v[3].w};
    const Conv16 cv = convert16(e);
    if (store) {
        unsigned char* col = xs + (size_t)(G >> 4) * kQ6Col;
        const int g = G & 15;
        const int h = g >> 3;
        const int t = (g >> 1) & 3;
        const int a = g & 1;
        const int quad = 2 * h + a;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            *reinterpret_cast<uint4*>(col + kQ6Digits + quad * 256 + (4 * t + u) * 16) =
                make_uint4(cv.plane[0][u], cv.plane[1][u], cv.plane[2][u], cv.plane[3][u]);
        }
        *reinterpret_cast<double*>(col + kQ6Sum + (quad * 4 + t) * 8) = cv.xsum16;
        if (a == 0) {
            *reinterpret_cast<double*>(col + kQ6Scale + (h * 4 + t) * 8) = grid_scale(cv.sigma);
        }
        if (g == 0) {
            *reinterpret_cast<uint32_t*>(col + kQ6Word) = (uint32_t)cv.total;
        }
        store_corrections(col + kQ6List, cv, e, 16 * g);
    }
}

// 16 bytes starting `sh` (0 or 2) bytes into the dword at p (4-byte
// aligned): five aligned dword reads, shifted.
__device__ __forceinline__ void read16_shifted(const unsigned char* p, uint32_t sh, uint32_t (&o)[4])
{
    const uint32_t* d = reinterpret_cast<const uint32_t*>(p);
    const uint32_t d0 = d[0], d1 = d[1], d2 = d[2], d3 = d[3], d4 = d[4];
    o[0] = __builtin_amdgcn_alignbyte(d1, d0, sh);
    o[1] = __builtin_amdgcn_alignbyte(d2, d1, sh);
    o[2] = __builtin_amdgcn_alignbyte(d3, d2, sh);
    o[3] = __builtin_amdgcn_alignbyte(d4, d3, sh);
}

// Code dword u of group t (t, u < 4), by masks (no indexed register read).
__device__ __forceinline__ uint32_t pick_q6_code(const int (&c)[4][4], int t, int u)
{
    uint32_t r = 0;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
            r |= (uint32_t)c[tt][uu] & (0u - (uint32_t)(tt == t && uu == u));
        }
    }
    return r;
}

// NW waves; UB = 64 or 128 (w 128-byte aligned: whole lines): the bytes of
// a row one load instruction reads; BB = 128 or 256: the bytes of a row per
// batch (256 only where no row has a phase); XC groups of 16 x per thread.
template <int NW, int UB, int BB, int XC>
__global__ void __launch_bounds__(NW * 64)
q6k_gemv_kernel(const uint8_t* __restrict__ w, const float* __restrict__ x,
                float* __restrict__ y, int n, int S, long long row_stride, int rows_per_block,
                int ncg)
{
    static_assert(UB == 64 || UB == 128, "unit");
    static_assert(BB == 128 || BB == 256, "batch");
    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int quad = lane >> 4;
    const int j = lane & 15;
    const int hq = quad >> 1;
    const int aq = quad & 1;
    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ntiles = (rows_here + 15) >> 4;
    const int ntasks = ntiles * ncg;
    const int my_tasks = ntasks > wave ? (ntasks - wave + NW - 1) / NW : 0;

    const size_t xbytes = (size_t)S * kQ6Col;
    unsigned char* ring = smem + xbytes + wave * kQ6Wave;
    double* ypart = reinterpret_cast<double*>(smem + xbytes + NW * kQ6Wave);

    // load role: LPR lanes per row and instruction; a batch is BB bytes of
    // each of the tile's 16 rows, NI instructions
    constexpr int LPR = UB / 16;
    constexpr int NI = BB / 64;
    const int lrow = lane / LPR;
    const int lpiece = lane % LPR;
    // instruction i (< NI) of a batch: the tile row it reads (the lane's
    // first or second row, i & 1, for line units) and its byte offset
    // within the batch
    auto ins_row = [&](int i) __attribute__((always_inline)) {
        return UB == 64 ? lrow : 8 * (i & 1) + lrow;
    };
    auto ins_off = [&](int i) __attribute__((always_inline)) {
        return UB == 64 ? 64 * i + 16 * lpiece : 128 * (i >> 1) + 16 * lpiece;
    };
    // a row's batches start on a line (UB = 128; w is 128-byte aligned) or
    // on its first 16-byte piece: the row's bytes sit `phase` bytes into
    // its ring, at most kPhaseMax.  When the row stride is a multiple of
    // kAlign every row starts on a line, and a task's origin B0 is aligned
    // down to one too, so no row has a phase
    constexpr uint32_t kAlign = UB == 128 ? 128u : 16u;
    const bool aligned_rows = ((uint64_t)row_stride & (kAlign - 1u)) == 0;
    const uint32_t kPhaseMax = aligned_rows ? 0u : kAlign - 16u;
    const uint32_t kOriginMask = aligned_rows ? ~(kAlign - 1u) : ~15u;

    // x: all of it converted into LDS, the first batches of weights already
    // in flight
    const int ngroups = S * 16;
    float4 xv[XC][4];
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int G = min(tid + i * NW * 64, ngroups - 1);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            xv[i][t] = reinterpret_cast<const float4*>(x)[4 * G + t];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // task q of this wave (clamped into its tasks): tile, columns [c0, c1)
    auto task_cols = [&](int q, int& tile, int& c0, int& c1) __attribute__((always_inline)) {
        const int qc = max(0, min(q, my_tasks - 1));
        const int task = min(wave + qc * NW, max(ntasks - 1, 0));
        tile = task / ncg;
        const int cg = task % ncg;
        c0 = (int)((long long)cg * S / ncg);
        c1 = (int)((long long)(cg + 1) * S / ncg);
    };
    // per task: for the two rows the lane loads, the byte offset from w of
    // its batch 0 (the row's bytes from the task's origin B0 at or before
    // column c0, aligned down to kAlign) and the end of the 16-byte pieces
    // holding the task's bytes; the phase of the lane's compute row j
    struct TaskGeo {
        uint64_t a[2], lim[2];
        uint32_t B0, pj;
    };
    auto task_geo = [&](int q) __attribute__((always_inline)) {
        int tile, c0, c1;
        task_cols(q, tile, c0, c1);
        TaskGeo g;
        g.B0 = (210u * (uint32_t)c0) & kOriginMask;
        const uint32_t last = (210u * (uint32_t)c1 - 1u) & ~15u;
        const bool past = q >= my_tasks;        // the prefetch after the wave's last task
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = min(tile * 16 + ins_row(h), rows_here - 1);
            const uint64_t rb = (uint64_t)(row0 + r) * (uint64_t)row_stride;
            g.a[h] = (rb + g.B0) & ~(uint64_t)(kAlign - 1u);
            g.lim[h] = past ? 0u : rb + last + 16u;     // pieces below it are the task's
        }
        const int rj = min(tile * 16 + j, rows_here - 1);
        g.pj = (uint32_t)(((uint64_t)(row0 + rj) * (uint64_t)row_stride + g.B0) &
                          (uint64_t)(kAlign - 1u));
        return g;
    };
    constexpr int kNBF = 512 / BB;           // batches in flight per wave (and ring slots)
    uint4 regs[kNBF][NI];
    // a piece past the task's bytes (the surplus batches, the prefetch after
    // the last task) reads 16 bytes of x instead: cached, so it costs no HBM
    // traffic (x holds k * 4 >= 1024 bytes; a select, not a branch)
    const uint64_t dx = (uint64_t)(reinterpret_cast<const uint8_t*>(x) - w) + 16u * (uint32_t)lane;
    auto issue = [&](const TaskGeo& g, int b, int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint64_t o = g.a[i & 1] + (uint32_t)BB * (uint32_t)b + (uint32_t)ins_off(i);
            const uint64_t off = o < g.lim[i & 1] ? o : dx;
            regs[slot][i] = load_line_nt(w + off);
        }
    };
    auto issue_first = [&](const TaskGeo& g) __attribute__((always_inline)) {
        static_for<kNBF>([&](auto I) __attribute__((always_inline)) {
            issue(g, decltype(I)::value, decltype(I)::value);
        });
    };
    // the first batches of the wave's first task go out before the
    // conversion.  No load sits behind a branch (a wave without tasks loads
    // from its clamped task too): the compiler's counter waits then let
    // the conversion wait for x alone, and the stream keep every batch in
    // flight
    TaskGeo geo = task_geo(0);
    issue_first(geo);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < XC; ++i) {
        const int G = tid + i * NW * 64;
        convert_group_q6(xv[i], G, G < ngroups, smem);
    }
    __syncthreads();

    unsigned char* rr = ring + j * kQ6Row;      // the lane's row in the ring (compute role)
    double acc = 0.0;
    uint64_t flags[2] = {0, 0};                 // columns of the task with exact terms (S <= 128)

    // column c of the task (origin B0, the lane's row at phase pj): its 210
    // bytes are in the ring
    auto column = [&](int c, uint32_t B0, uint32_t pj) __attribute__((always_inline)) {
        const unsigned char* col = smem + (size_t)c * kQ6Col;
        const uint4 xd = *reinterpret_cast<const uint4*>(col + kQ6Digits + quad * 256 + j * 16);
        const double2 xi01 = *reinterpret_cast<const double2*>(col + kQ6Sum + quad * 32);
        const double2 xi23 = *reinterpret_cast<const double2*>(col + kQ6Sum + quad * 32 + 16);
        const double2 s01 = *reinterpret_cast<const double2*>(col + kQ6Scale + hq * 32);
        const double2 s23 = *reinterpret_cast<const double2*>(col + kQ6Scale + hq * 32 + 16);
        const uint32_t cnt = *reinterpret_cast<const uint32_t*>(col + kQ6Word);
        const uint32_t rel = 210u * (uint32_t)c - B0;
        const uint32_t r0 = (pj + rel) & (uint32_t)(kQ6Ring - 1);
        const uint32_t sh = rel & 3u;                // wave-uniform (pj % 16 == 0): 0 or 2
        auto at = [&](uint32_t f) __attribute__((always_inline)) {
            return rr + ((r0 + f) & (uint32_t)(kQ6Ring - 4));
        };
        uint32_t A[4], B[4], H[4];
        read16_shifted(at(64u * hq + 16u * aq), sh, A);
        read16_shifted(at(64u * hq + 32u + 16u * aq), sh, B);
        read16_shifted(at(128u + 32u * hq + 16u * aq), sh, H);
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(at(192u + 8u * hq));
        const uint32_t sw0 = __builtin_amdgcn_alignbyte(sp[1], sp[0], sh);
        const uint32_t sw1 = __builtin_amdgcn_alignbyte(sp[2], sp[1], sh);
        const uint32_t dw = *reinterpret_cast<const uint32_t*>(at(208u));
        const uint16_t dbits = (uint16_t)(dw >> (8u * sh));
        const float d = (float)__builtin_bit_cast(_Float16, dbits);
        // codes q (0..63) of group t, dword u: elements 16 a + 4 u .. + 3
        int cq[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            cq[0][u] = (int)((A[u] & 0x0F0F0F0Fu) | ((H[u] << 4) & 0x30303030u));
            cq[1][u] = (int)((B[u] & 0x0F0F0F0Fu) | ((H[u] << 2) & 0x30303030u));
            cq[2][u] = (int)(((A[u] >> 4) & 0x0F0F0F0Fu) | (H[u] & 0x30303030u));
            cq[3][u] = (int)(((B[u] >> 4) & 0x0F0F0F0Fu) | ((H[u] >> 2) & 0x30303030u));
        }
        int t01[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int t23[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        q6_dot_pair<0>(xd, cq[0], cq[1], t01);
        q6_dot_pair<1>(xd, cq[2], cq[3], t23);
        // scales 8 h + 2 t + a: bytes a, a + 2 of sw0 (t = 0, 1) and of sw1
        // (signed bytes: a plain int8_t conversion, so the sign survives)
        const uint32_t sa = 8u * (uint32_t)aq;
        float D[4];
        D[0] = d * (float)(int)(int8_t)(uint8_t)(sw0 >> sa);
        D[1] = d * (float)(int)(int8_t)(uint8_t)(sw0 >> (sa + 16u));
        D[2] = d * (float)(int)(int8_t)(uint8_t)(sw1 >> sa);
        D[3] = d * (float)(int)(int8_t)(uint8_t)(sw1 >> (sa + 16u));
        const double XI[4] = {xi01.x, xi01.y, xi23.x, xi23.y};
        const double SC[4] = {s01.x, s01.y, s23.x, s23.y};
        const double T0 = digits_exact(t01[0], t01[1], t01[2], t01[3]);
        const double T1 = digits_exact(t01[4], t01[5], t01[6], t01[7]);
        const double T2 = digits_exact(t23[0], t23[1], t23[2], t23[3]);
        const double T3 = digits_exact(t23[4], t23[5], t23[6], t23[7]);
        // d sc (T - 32 XI): 32 d sc is exact, so subblock_term rounds once
        acc = subblock_term(acc, D[0], T0, 32.0f * D[0], XI[0], SC[0]);
        acc = subblock_term(acc, D[1], T1, 32.0f * D[1], XI[1], SC[1]);
        acc = subblock_term(acc, D[2], T2, 32.0f * D[2], XI[2], SC[2]);
        acc = subblock_term(acc, D[3], T3, 32.0f * D[3], XI[3], SC[3]);
        // a column with elements the digits leave out: its exact terms come
        // after the stream (correct_column), so this code stays small
        const uint32_t ncorr = __builtin_amdgcn_readfirstlane(cnt);
        if (ncorr != 0u) {
            flags[c >> 6] |= 1ull << (c & 63);
        }
    };

    // the exact terms fl32(d sc (q - 32)) x (in f64, the oracle's arithmetic)
    // of the elements of column c that the digits leave out, for the lane's
    // row of `tile`: the column's bytes read again from global memory (five
    // aligned dwords per 16-byte field, shifted; d by a 16-bit load)
    auto correct_column = [&](int c, int tile) __attribute__((always_inline)) {
        const unsigned char* col = smem + (size_t)c * kQ6Col;
        const uint32_t ncorr =
            __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(col + kQ6Word));
        const double2 s01 = *reinterpret_cast<const double2*>(col + kQ6Scale + hq * 32);
        const double2 s23 = *reinterpret_cast<const double2*>(col + kQ6Scale + hq * 32 + 16);
        const double SC[4] = {s01.x, s01.y, s23.x, s23.y};
        const int rj = min(tile * 16 + j, rows_here - 1);
        const uint8_t* sb = w + (uint64_t)(row0 + rj) * (uint64_t)row_stride + 210u * (uint32_t)c;
        const uint32_t sh = (210u * (uint32_t)c) & 3u;
        const uint8_t* sb4 = sb - sh;                   // 4-byte aligned
        uint32_t A[4], B[4], H[4];
        read16_shifted(sb4 + 64u * hq + 16u * aq, sh, A);
        read16_shifted(sb4 + 64u * hq + 32u + 16u * aq, sh, B);
        read16_shifted(sb4 + 128u + 32u * hq + 16u * aq, sh, H);
        const uint32_t* sp = reinterpret_cast<const uint32_t*>(sb4 + 192u + 8u * hq);
        const uint32_t sw0 = __builtin_amdgcn_alignbyte(sp[1], sp[0], sh);
        const uint32_t sw1 = __builtin_amdgcn_alignbyte(sp[2], sp[1], sh);
        const uint16_t dbits = *reinterpret_cast<const uint16_t*>(sb + 208);
        const float d = (float)__builtin_bit_cast(_Float16, dbits);
        int cq[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            cq[0][u] = (int)((A[u] & 0x0F0F0F0Fu) | ((H[u] << 4) & 0x30303030u));
            cq[1][u] = (int)((B[u] & 0x0F0F0F0Fu) | ((H[u] << 2) & 0x30303030u));
            cq[2][u] = (int)(((A[u] >> 4) & 0x0F0F0F0Fu) | (H[u] & 0x30303030u));
            cq[3][u] = (int)(((B[u] >> 4) & 0x0F0F0F0Fu) | ((H[u] >> 2) & 0x30303030u));
        }
        const uint32_t sa = 8u * (uint32_t)aq;
        float D[4];
        D[0] = d * (float)(int)(int8_t)(uint8_t)(sw0 >> sa);
        D[1] = d * (float)(int)(int8_t)(uint8_t)(sw0 >> (sa + 16u));
        D[2] = d * (float)(int)(int8_t)(uint8_t)(sw1 >> sa);
        D[3] = d * (float)(int)(int8_t)(uint8_t)(sw1 >> (sa + 16u));
        if (ncorr <= (uint32_t)kCorr) {
            for (uint32_t k = 0; k < ncorr; ++k) {
                const Corr cr = *reinterpret_cast<const Corr*>(col + kQ6List + k * 8);
                const int e = __builtin_amdgcn_readfirstlane((int)cr.e);
                const float xe = __builtin_bit_cast(
                    float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, cr.x)));
                const int te = (e >> 5) & 3;
                const int ie = e & 15;
                const uint32_t q = (pick_q6_code(cq, te, ie >> 2) >> (8 * (ie & 3))) & 63u;
                const float De = te == 0 ? D[0] : te == 1 ? D[1] : te == 2 ? D[2] : D[3];
                const float wv = De * (float)((int)q - 32);
                const double tv = (double)wv * (double)xe;
                const bool mine = (e >> 7) == hq && ((e >> 4) & 1) == aq;
                acc = mine ? acc + tv : acc;
            }
        } else {
            const float* xg = x + (size_t)c * 256 + 128 * hq + 16 * aq;
#pragma nounroll
            for (int te = 0; te < 4; ++te) {
                const float4* src = reinterpret_cast<const float4*>(xg + 32 * te);
                float4 xe4[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    xe4[u] = src[u];
                }
                const int sigma = grid_sigma_of(te == 0 ? SC[0] : te == 1 ? SC[1]
                                                : te == 2 ? SC[2] : SC[3]);
                const float De = te == 0 ? D[0] : te == 1 ? D[1] : te == 2 ? D[2] : D[3];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t cw = pick_q6_code(cq, te, u);
                    const float xs4[4] = {xe4[u].x, xe4[u].y, xe4[u].z, xe4[u].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t uu;
                        int cert;
                        grid_element(xs4[i], sigma, uu, cert);
                        const int q = (int)((cw >> (8 * i)) & 63u);
                        const float wv = De * (float)(q - 32);
                        const double tv = (double)wv * (double)xs4[i];
                        acc = cert ? acc : acc + tv;
                    }
                }
            }
        }
    };

    for (int q = 0; q < my_tasks; ++q) {
        int tile, c0, c1;
        task_cols(q, tile, c0, c1);
        const uint32_t B0 = geo.B0;
        // batches, in whole groups of kNBF (the surplus ones read x and
        // complete no column)
        const int nb = (int)((210u * (uint32_t)c1 - B0 + kPhaseMax + BB - 1u) / (uint32_t)BB);
        const int nbr = (nb + kNBF - 1) / kNBF * kNBF;
        int c = c0;
        // batch b (register and ring slot b % kNBF) into the ring, batch
        // b + kNBF out into its registers, then every column whose bytes
        // are in the ring for every row of the tile.  The slot written next
        // holds none of a column not yet computed: with BB = 128 (four
        // slots) such a column starts past 128 (b + 1) - 210 - 112, beyond
        // batch b - 3; with BB = 256 (two slots; no row has a phase) past
        // 256 (b + 1) - 210, inside batch b.
        auto consume = [&](int b, auto sc) __attribute__((always_inline)) {
            constexpr int sl = decltype(sc)::value;
            constexpr int rs = sl;                 // ring slot (kNBF slots of BB bytes)
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int o = rs * BB + ins_off(i);
                unsigned char* wr = ring + ins_row(i) * kQ6Row;
                *reinterpret_cast<uint4*>(wr + o) = regs[sl][i];
                if (rs == 0 && o < 32) {
                    *reinterpret_cast<uint4*>(wr + kQ6Ring + o) = regs[sl][i];
                }
            }
            __builtin_amdgcn_sched_barrier(0x000F);
            issue(geo, b + kNBF, sl);
            const uint32_t have = (uint32_t)BB * (uint32_t)(b + 1);
            while (c < c1 && 210u * (uint32_t)(c + 1) - B0 + kPhaseMax <= have) {
                column(c, B0, geo.pj);
                ++c;
            }
        };
        for (int b = 0; b < nbr; b += kNBF) {
            static_for<kNBF>([&](auto I) __attribute__((always_inline)) {
                consume(b + decltype(I)::value, I);
            });
        }
        // the next task's first batches (after the last task: x)
        geo = task_geo(q + 1);
        issue_first(geo);
        // the task's columns with elements the digits leave out
        for (int h = 0; h < 2; ++h) {
            while (flags[h] != 0u) {
                const int cf = 64 * h + __builtin_ctzll(flags[h]);
                flags[h] &= flags[h] - 1u;
                correct_column(cf, tile);
            }
        }
        // the rows of the task: four quadrant lanes per row
        double v = acc;
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        acc = 0.0;
        const int r = tile * 16 + j;
        if (quad == 0 && r < rows_here) {
            if (ncg == 1) {
                y[row0 + r] = (float)v;
            } else {
                const int task = wave + q * NW;
                ypart[(task % ncg) * rows_per_block + r] = v;
            }
        }
    }
    // drain: the surplus loads of the last task complete before the wave
    // ends (their registers are otherwise dead)
    __builtin_amdgcn_s_waitcnt(0);

    if (ncg > 1) {
        __syncthreads();
        for (int i = tid; i < rows_here; i += NW * 64) {
            double a = 0.0;
            for (int g = 0; g < ncg; ++g) {
                a += ypart[g * rows_per_block + i];
            }
            y[row0 + i] = (float)a;
        }
    }
}

// Dequantize: one thread per 16 weights (one scale); w = d sc (q - 32),
// exact in f32 (T = float), or that weight rounded to fp16 to nearest even
// (T = _Float16: the mirror).
template <typename T>
__global__ void __launch_bounds__(256)
q6k_dequant_kernel(const uint8_t* __restrict__ w, T* __restrict__ out, int64_t n, int S,
                   long long row_stride)
{
    const int64_t gidx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = n * (int64_t)S * 16;
    if (gidx >= total) {
        return;
    }
    const int g = (int)(gidx & 15);
    const int64_t sbi = gidx >> 4;
    const int64_t r = sbi / S;
    const int s = (int)(sbi % S);
    const uint8_t* blk = w + r * row_stride + (int64_t)s * 210;
    const int h = g >> 3;
    const int t = (g >> 1) & 3;
    const int l0 = 16 * (g & 1);
    const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(blk[208] | (blk[209] << 8)));
    const float D = d * (float)(int8_t)blk[192 + g];
    float o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint8_t lb = blk[64 * h + 32 * (t & 1) + l0 + i];
        const uint8_t hb = blk[128 + 32 * h + l0 + i];
        const int lo = t < 2 ? (lb & 15) : (lb >> 4);
        const int hi = (hb >> (2 * t)) & 3;
        o[i] = D * (float)(lo + 16 * hi - 32);
    }
    T* dst = out + r * (int64_t)S * 256 + (int64_t)s * 256 + 16 * g;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        dst[i] = (T)o[i];
    }
}

template <int NW, int UB, int BB>
static hipError_t launch_q6k_u(const Q6kPlan& p, const uint8_t* w, const float* x, float* y,
                               hipStream_t stream)
{
    const int per = (p.S * 16 + NW * 64 - 1) / (NW * 64);
#define Q6K_LAUNCH(XC)                                                                       \
    hipLaunchKernelGGL((q6k_gemv_kernel<NW, UB, BB, XC>), dim3(p.grid), dim3(NW * 64),         \
                       p.lds_bytes, stream, w, x, y, p.n, p.S, (long long)p.row_stride,        \
                       p.rows_per_block, p.ncg)
    if (per <= 1) {
        Q6K_LAUNCH(1);
    } else if (per <= 2) {
        Q6K_LAUNCH(2);
    } else if (per <= 4) {
        Q6K_LAUNCH(4);
    } else {
        return hipErrorInvalidValue;
    }
#undef Q6K_LAUNCH
    return hipGetLastError();
}

template <int NW>
static hipError_t launch_q6k_w(const Q6kPlan& p, const uint8_t* w, const float* x, float* y,
                               hipStream_t stream)
{
    if (p.unit == 64) {
        return launch_q6k_u<NW, 64, 256>(p, w, x, y, stream);
    }
    return p.batch == 256 ? launch_q6k_u<NW, 128, 256>(p, w, x, y, stream)
                          : launch_q6k_u<NW, 128, 128>(p, w, x, y, stream);
}

hipError_t launch_q6k_gemv(const Q6kPlan& p, const void* w, const float* x, float* y,
                           hipStream_t stream)
{
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    if (p.unit == 64 && p.batch != 256) {
        return hipErrorInvalidValue;
    }
    if (p.waves_per_block == 8) {
        return launch_q6k_w<8>(p, wb, x, y, stream);
    }
    if (p.waves_per_block == 4) {
        return launch_q6k_w<4>(p, wb, x, y, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_q6k_dequant(const void* w, float* out, int64_t n, int S, int64_t row_stride,
                              hipStream_t stream)
{
    const int64_t total = n * (int64_t)S * 16;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(q6k_dequant_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const uint8_t*>(w), out, n, S, (long long)row_stride);
    return hipGetLastError();
}

hipError_t launch_q6k_dequant_f16(const void* w, void* out, int64_t n, int S, int64_t row_stride,
                                  hipStream_t stream)
{
    const int64_t total = n * (int64_t)S * 16;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(q6k_dequant_kernel<_Float16>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, static_cast<const uint8_t*>(w), static_cast<_Float16*>(out), n, S,
                       (long long)row_stride);
    return hipGetLastError();
}

size_t q6k_lds_bytes(int S, int waves, int rows_per_block, int ncg)
{
    return (size_t)S * kQ6Col + (size_t)waves * kQ6Wave +
           (ncg > 1 ? (size_t)rows_per_block * ncg * 8 : 0);
}

}  // namespace q4k

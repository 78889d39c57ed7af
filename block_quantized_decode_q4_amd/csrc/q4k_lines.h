// q4k_lines.h -- the line stream shared by the line-streamed GEMV kernels
// (q4k_dpp.hip: vector-ALU dot products; q4k_mfma.hip: matrix cores).
// Internal.
//
// A wave reads its 16 rows of weights in whole 128-byte lines (eight lanes
// per row and line, two instructions per line index), non-temporally, and
// writes each line into a per-wave ring of two lines per row in LDS, from
// which the lanes take the superblocks in whatever layout their arithmetic
// wants.  Every weight byte is fetched once, by one instruction that uses its
// whole cache line -- the access the memory system streams fastest.  Eight
// superblocks of a row are nine lines (8 x 144 = 9 x 128), so rows must be
// 128-byte aligned and hold a multiple of eight superblocks.  Superblock c'
// of a slab of eight uses lines c' and c'+1 of the slab; a ring of P line
// slots in registers (P = 3, or 9: a whole slab) keeps P lines in flight per
// wave.  A wave walks its tasks (tile of 16 rows, group of slabs) as one
// stream, so the loads of the next task go out while the current one
// finishes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace q4k {

constexpr int kRingRow = 2 * 128 + 16;        // two lines per row, padded

// a step that takes (c, cend, cn, rr, b0, cp, valid): see line_stream
template <typename Step>
constexpr bool kLookAhead =
    std::is_invocable_v<Step&, int, int, int, unsigned char*, uint32_t, int, bool>;
constexpr int kRingWave = 16 * kRingRow;

// a step that takes (c, rr, b0, corr) with corr a std::integral_constant:
// the stream calls it with true only for slabs whose slab_flag is set, so a
// step keeps a rarely taken path out of the other slabs' code
template <typename Step>
constexpr bool kFlagged =
    std::is_invocable_v<Step&, int, unsigned char*, uint32_t, std::true_type>;

struct NoSlabFlag {
    __device__ bool operator()(int) const { return false; }
};

// f(std::integral_constant<int, i>()) for i = 0 .. N-1, each call inlined:
// a loop whose body must see its index as a constant, whatever its size
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>()), ...);
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>());
}

__device__ __forceinline__ uint4 load_line_nt(const uint8_t* p)
{
    typedef unsigned v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The line stream shared by the line-streamed kernels.  Work: the
// workgroup's rows in 16-row tiles, each row in slabs of eight superblocks;
// a task is (tile, group of slabs_per_task slabs) and wave w takes tasks w,
// w + NW, ...  Calls, in order: issue_x() (the x loads), the first P lines
// of weights go out, convert_x() (x into LDS), a workgroup barrier, then
// step(c, rr, b0) for every superblock column c of the wave's tasks in order
// (rr: the ring row of the lane's tile row j, b0 = 144 (c mod 8): the
// superblock's byte offset in that row's two-line ring window, mod 256; a
// compile-time constant) and task_end(task) after each task's last slab.
// A look-ahead step, step(c, cend, cn, rr, b0, cp, valid), also gets the
// end cend of the columns of c's slab (or task), the first column cn of the
// wave's next slab (task; its last one again after the last), c's position
// cp in its slab and whether c is a column of the row at all (rows of
// partial slabs: the positions past the row's end are passed too, invalid,
// so that a step can keep state that cycles with cp).
// Line l of every slab goes to ring slot l mod 2: the previous slab's last
// line (slot 0) is dead once its last superblock has been read, and the
// wave's LDS accesses complete in order.
template <int NW, int P, typename IssueX, typename ConvertX, typename Step, typename TaskEnd,
          typename SlabFlag = NoSlabFlag, bool PREPUT = false, bool ONEBODY = false>
__device__ __forceinline__ void line_stream(const uint8_t* __restrict__ w,
                                            const float* __restrict__ x, int n, int S,
                                            int rows_per_block, int slabs_per_task,
                                            unsigned char* ring, IssueX issue_x,
                                            ConvertX convert_x, Step step, TaskEnd task_end,
                                            SlabFlag slab_flag = SlabFlag())
{
    static_assert(P == 3 || P == 9, "line slots must divide the nine lines of a slab");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int j = lane & 15;
    // load role: eight lanes per row and line
    const int lrow = lane >> 3;
    const int lunit = lane & 7;

    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ntiles = (rows_here + 15) >> 4;
    const int ncg = (S >> 3) / slabs_per_task;
    const int ntasks = ntiles * ncg;
    const int my_tasks = ntasks > wave ? (ntasks - wave + NW - 1) / NW : 0;
    const int my_slabs = my_tasks * slabs_per_task;
    const size_t row_bytes = (size_t)S * 144;

    // slab sig of this wave -> (tile, absolute slab); clamped into the
    // wave's slabs (and into the block's tasks for a wave without any), so
    // every prefetch address is valid and no load sits behind a branch
    auto slab_of = [&](int sig, int& tile, int& slab) __attribute__((always_inline)) {
        sig = max(0, min(sig, my_slabs - 1));
        const int task = min(wave + (sig / slabs_per_task) * NW, ntasks - 1);
        tile = task / ncg;
        slab = (task % ncg) * slabs_per_task + sig % slabs_per_task;
    };
    // the byte offsets from w of line 0 of slab sig for rows lrow and
    // 8 + lrow (the lane's 16 bytes of them), and the line stride; past the
    // wave's last slab the prefetch reads a 128-byte line of x instead, with
    // stride 0 (cached, so the surplus loads cost no HBM traffic; each wave
    // takes its own line, or the tails of all waves would queue on one L2
    // channel).  The choice is a mask on the byte offset from w: a select of
    // two pointers makes the compiler branch around the address arithmetic,
    // which costs registers across the unrolled slab.  Computed once per
    // slab, so a line costs one 64-bit add per row.
    const int xlines = S * 8;                        // 128-byte lines of one x vector
    const uint64_t dx = (uint64_t)(reinterpret_cast<const uint8_t*>(x) - w) +
                        (uint64_t)((blockIdx.x * NW + wave) % xlines) * 128u +
                        16u * (uint32_t)lunit;
    struct SlabBase {
        uint64_t b[2];
        uint32_t stride;
    };
    auto slab_base = [&](int sig) __attribute__((always_inline)) {
        int tile, slab;
        slab_of(sig, tile, slab);
        const bool past = sig >= my_slabs;                          // wave-uniform
        const uint64_t mask = past ? ~0ull : 0ull;
        SlabBase sb;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = min(tile * 16 + 8 * h + lrow, rows_here - 1);
            const uint64_t full = (uint64_t)(row0 + r) * row_bytes + (uint64_t)slab * 1152u +
                                  16u * (uint32_t)lunit;
            sb.b[h] = (full & ~mask) | (dx & mask);
        }
        sb.stride = past ? 0u : 128u;
        return sb;
    };
    auto line_ptrs = [&](const SlabBase& sb, int l, const uint8_t** p) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            p[h] = w + sb.b[h] + (uint64_t)(sb.stride * (uint32_t)l);
        }
    };

    // x loads first, then the first lines of weights, then the conversion:
    // waiting for x (the counter of loads returns in order) then leaves the
    // weight lines in flight.  No wave sends weight loads before every wave
    // of the workgroup has sent its x loads (a barrier with no wait for
    // memory), so x is not queued behind the workgroup's own weight lines.
    issue_x();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    uint4 lines[P][2];
    {
        const SlabBase sb0 = slab_base(0);
#pragma unroll
        for (int l = 0; l < P; ++l) {
            const uint8_t* p[2];
            line_ptrs(sb0, l, p);
            lines[l][0] = load_line_nt(p[0]);
            lines[l][1] = load_line_nt(p[1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        convert_x();
        if constexpr (PREPUT && P == 3) {
            // lines 0 and 1 of the first slab into the ring now, their
            // register slots refilled with lines 3 and 4 before the barrier
#pragma unroll
            for (int l = 0; l < 2; ++l) {
                const uint32_t lpos = (uint32_t)l * 128u + 16u * (uint32_t)lunit;
                *reinterpret_cast<uint4*>(ring + lrow * kRingRow + lpos) = lines[l][0];
                *reinterpret_cast<uint4*>(ring + (8 + lrow) * kRingRow + lpos) = lines[l][1];
                __builtin_amdgcn_sched_barrier(0x000F);
                const uint8_t* p[2];
                line_ptrs(sb0, l + P, p);
                lines[l][0] = load_line_nt(p[0]);
                lines[l][1] = load_line_nt(p[1]);
            }
        }
    }
    __syncthreads();

    // Waves w and w + 4 of an 8-wave workgroup share a SIMD, and with equal
    // priority the older (w) wins every issue arbitration: with equal work
    // the younger ends about 1 us later (wave timestamps, LM head), and the
    // SIMD finishes on one wave.  With equal work of at least two slabs the
    // younger raises its priority for the stream (the older has got ahead
    // during the x stage), which evens out the end times (LM head -0.2 us,
    // 128256 x 4096 -0.35 us; one slab each: no gain, so left alone).  Set
    // once, outside the stream, so the stream's code is unchanged.
    if (NW == 8 && wave >= 4 && my_slabs >= 2 &&
        (ntasks - (wave - 4) + NW - 1) / NW == my_tasks) {
        __builtin_amdgcn_s_setprio(1);
    }
    auto slab_iter = [&](int sig, auto first) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first)::value;
        int tile, slab, tile_n, slab_n;
        slab_of(sig, tile, slab);
        slab_of(sig + 1, tile_n, slab_n);      // clamped: the last slab again at the end
        const SlabBase cur = slab_base(sig);
        const SlabBase nxt = slab_base(sig + 1);
        // line l (compile-time) of the slab into the ring, and its slot
        // refilled with line l + P
        auto put = [&](auto lc) __attribute__((always_inline)) {
            constexpr int l = decltype(lc)::value;
            constexpr int slot = l % P;
            const uint32_t lpos = (uint32_t)(l & 1) * 128u + 16u * (uint32_t)lunit;
            *reinterpret_cast<uint4*>(ring + lrow * kRingRow + lpos) = lines[slot][0];
            *reinterpret_cast<uint4*>(ring + (8 + lrow) * kRingRow + lpos) = lines[slot][1];
            // memory operations stay in order here (the refill after the
            // write of its slot); arithmetic may move across
            __builtin_amdgcn_sched_barrier(0x000F);
            constexpr int ln = l + P;                  // refill: P lines ahead
            const uint8_t* p[2];
            line_ptrs(ln >= 9 ? nxt : cur, ln >= 9 ? ln - 9 : ln, p);
            lines[slot][0] = load_line_nt(p[0]);
            lines[slot][1] = load_line_nt(p[1]);
        };
        // superblock cp (compile-time) of the slab: lines 0 and 1 before
        // the first, then line cp + 1; then the step on the ring of tile row
        // j (and, for a step that looks ahead, the end of this slab's columns
        // and the first column of the next slab).  Compile-time positions
        // keep every index into the line registers constant, however large
        // the step's body.
        auto slab_body = [&](auto corr) __attribute__((always_inline)) {
            static_for<8>([&](auto cpc) __attribute__((always_inline)) {
                constexpr int cp = decltype(cpc)::value;
                if constexpr (!(FIRST && cp == 0)) {
                    if constexpr (cp == 0) {
                        put(std::integral_constant<int, 0>());
                    }
                    put(std::integral_constant<int, cp + 1>());
                }
                if constexpr (kLookAhead<Step>) {
                    step(8 * slab + cp, 8 * slab + 8, 8 * slab_n, ring + j * kRingRow,
                         (uint32_t)(144 * cp), cp, true);
                } else if constexpr (kFlagged<Step>) {
                    step(8 * slab + cp, ring + j * kRingRow, (uint32_t)(144 * cp), corr);
                } else {
                    step(8 * slab + cp, ring + j * kRingRow, (uint32_t)(144 * cp));
                }
            });
        };
        if constexpr (kFlagged<Step> && ONEBODY) {
            // one body whose steps test their columns themselves: no join of
            // two bodies' line registers (whose copies wait for every load in
            // flight); measured faster with one slab per task
            (void)slab_flag;
            slab_body(std::true_type());
        } else if constexpr (kFlagged<Step>) {
            if (slab_flag(slab)) {
                slab_body(std::true_type());
            } else {
                slab_body(std::false_type());
            }
        } else {
            slab_body(std::false_type());
        }
        if (sig % slabs_per_task == slabs_per_task - 1) {
            task_end(wave + (sig / slabs_per_task) * NW);
        }
    };
    int sig0 = 0;
    if constexpr (PREPUT && P == 3) {
        if (my_slabs > 0) {
            slab_iter(0, std::true_type());
            sig0 = 1;
        }
    }
    for (int sig = sig0; sig < my_slabs; ++sig) {
        slab_iter(sig, std::false_type());
    }
}

constexpr int kRing4Row = 4 * 128 + 16;       // four lines per row, padded
constexpr int kRing4Wave = 16 * kRing4Row;

// The line stream for rows of any whole number of superblocks: S % 8 may be
// non-zero, so a row starts on any 16-byte boundary of a line.  A 16-row
// tile is 18 S lines, so tiles start on a line (w 128-byte aligned) and row
// j of every tile starts (144 S j) mod 128 bytes into its first line.  Each
// row has a four-line ring.  A task (tile, slabs_per_task slabs) streams
// 9 slabs_per_task + 3 line indices per row: line 0, the nine further lines
// each slab reaches (a superblock that starts 112 bytes into a line ends in
// the next one, so the slab's reach is one line longer than when rows are
// aligned), and two surplus indices that keep a line's register slot equal
// to its index mod 3 from one task to the next.  A 16-byte piece past the
// row's bytes of the task is not loaded (the wave's line of x instead), so
// nothing beyond the matrix is read.  Superblock t of a task (t = 0 ..)
// needs lines floor(144 t / 128) .. floor((255 + 144 t) / 128) at most,
// three of the ring's four.  Calls as line_stream; step(c, rr, b0) gets
// b0 = 144 t, the byte offset within the task's ring window of 512 bytes
// before the lane adds its row's start offset, and runs only for the task's
// superblocks (the last slab of a row may hold fewer than eight).
template <int NW, typename IssueX, typename ConvertX, typename Step, typename TaskEnd,
          typename SlabFlag = NoSlabFlag>
__device__ __forceinline__ void line_stream_any(const uint8_t* __restrict__ w,
                                                const float* __restrict__ x, int n, int S,
                                                int rows_per_block, int slabs_per_task,
                                                unsigned char* ring, IssueX issue_x,
                                                ConvertX convert_x, Step step, TaskEnd task_end,
                                                SlabFlag slab_flag = SlabFlag())
{
    constexpr int P = 3;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int j = lane & 15;
    const int lrow = lane >> 3;
    const int lunit = lane & 7;

    const int row0 = blockIdx.x * rows_per_block;
    const int rows_here = min(rows_per_block, n - row0);
    const int ntiles = (rows_here + 15) >> 4;
    const int nslabs = (S + 7) >> 3;
    const int ncg = nslabs / slabs_per_task;
    const int ntasks = ntiles * ncg;
    const int my_tasks = ntasks > wave ? (ntasks - wave + NW - 1) / NW : 0;
    const int lpt = 9 * slabs_per_task + 3;          // line indices per task
    const size_t row_bytes = (size_t)S * 144;
    const int xlines = S * 8;
    const uint64_t dx = (uint64_t)(reinterpret_cast<const uint8_t*>(x) - w) +
                        (uint64_t)((blockIdx.x * NW + wave) % xlines) * 128u +
                        16u * (uint32_t)lunit;

    // task q of this wave (clamped into its tasks) -> (tile, column group,
    // superblocks)
    auto task_of = [&](int q, int& tile, int& cg, int& T) __attribute__((always_inline)) {
        const int qc = max(0, min(q, my_tasks - 1));
        const int task = min(wave + qc * NW, ntasks - 1);
        tile = task / ncg;
        cg = task % ncg;
        T = min(8 * slabs_per_task, S - 8 * cg * slabs_per_task);
    };
    // per task q and row (lrow, 8 + lrow): the byte offset from w of the
    // lane's 16 bytes of line 0, and the bound below which a line's piece
    // holds bytes of the row's task (128 L < lim); computed once per task.
    // x past the wave's tasks or the row's bytes of the task (a mask on the
    // byte offset from w, as in line_stream)
    struct TaskBase {
        uint64_t b[2];
        int lim[2];
    };
    auto task_base = [&](int q) __attribute__((always_inline)) {
        int tile, cg, T;
        task_of(q, tile, cg, T);
        const bool past = q >= my_tasks;                             // wave-uniform
        TaskBase tb;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = min(tile * 16 + 8 * h + lrow, rows_here - 1);
            const uint64_t start = (uint64_t)(row0 + r) * row_bytes;
            const int off = (int)((uint32_t)start & 127u);
            tb.b[h] = start - (uint64_t)off + (uint64_t)cg * slabs_per_task * 1152u +
                      16u * (uint32_t)lunit;
            tb.lim[h] = past ? 0 : off + 144 * T - 16 * lunit;
        }
        return tb;
    };
    auto line_ptrs = [&](const TaskBase& tb, int L, const uint8_t** p) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint64_t mask = 128 * L < tb.lim[h] ? 0ull : ~0ull;
            p[h] = w + (((tb.b[h] + 128u * (uint32_t)L) & ~mask) | (dx & mask));
        }
    };
    uint4 lines[P][2];
    // write line L = 9 s2 + X of the current task (bases cur, next task's
    // nxt) into the ring, refill its slot (X % 3) with the line three
    // indices on
    auto put = [&](const TaskBase& cur, const TaskBase& nxt, int s2, auto Xc) __attribute__((always_inline)) {
        constexpr int X = decltype(Xc)::value;
        constexpr int slot = X % P;
        const int L = 9 * s2 + X;
        const uint32_t lpos = ((uint32_t)L & 3u) * 128u + 16u * (uint32_t)lunit;
        *reinterpret_cast<uint4*>(ring + lrow * kRing4Row + lpos) = lines[slot][0];
        *reinterpret_cast<uint4*>(ring + (8 + lrow) * kRing4Row + lpos) = lines[slot][1];
        __builtin_amdgcn_sched_barrier(0x000F);
        const int ln = L + P;
        const uint8_t* p[2];
        line_ptrs(ln >= lpt ? nxt : cur, ln >= lpt ? ln - lpt : ln, p);
        lines[slot][0] = load_line_nt(p[0]);
        lines[slot][1] = load_line_nt(p[1]);
    };

    issue_x();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    {
        const TaskBase tb0 = task_base(0);
#pragma unroll
        for (int l = 0; l < P; ++l) {
            const uint8_t* p[2];
            line_ptrs(tb0, l, p);
            lines[l][0] = load_line_nt(p[0]);
            lines[l][1] = load_line_nt(p[1]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    convert_x();
    __syncthreads();

    for (int q = 0; q < my_tasks; ++q) {
        int tile, cg, T, tile_n, cg_n, T_n;
        task_of(q, tile, cg, T);
        task_of(q + 1, tile_n, cg_n, T_n);     // clamped: the last task again at the end
        const int c0 = 8 * cg * slabs_per_task;
        const int cn = 8 * cg_n * slabs_per_task;
        const TaskBase cur = task_base(q);
        const TaskBase nxt = task_base(q + 1);
        // superblock cp of slab s2 of the task, if the row has it
        auto stp = [&](int s2, int cp, auto corr) __attribute__((always_inline)) {
            const int c = c0 + 8 * s2 + cp;
            const uint32_t b0 = 1152u * (uint32_t)s2 + 144u * (uint32_t)cp;
            if constexpr (kLookAhead<Step>) {
                step(c, c0 + 8 * slabs_per_task, cn, ring + j * kRing4Row, b0, cp, 8 * s2 + cp < T);
            } else if constexpr (kFlagged<Step>) {
                if (8 * s2 + cp < T) step(c, ring + j * kRing4Row, b0, corr);
            } else {
                if (8 * s2 + cp < T) step(c, ring + j * kRing4Row, b0);
            }
        };
        auto slab_body = [&](int s2, auto corr) __attribute__((always_inline)) {
            // lines 9 s2 + 1 .. 9 s2 + 9: two before superblock 1 of the slab,
            // one before each other
            put(cur, nxt, s2, std::integral_constant<int, 1>());
            stp(s2, 0, corr);
            put(cur, nxt, s2, std::integral_constant<int, 2>());
            put(cur, nxt, s2, std::integral_constant<int, 3>());
            stp(s2, 1, corr);
            put(cur, nxt, s2, std::integral_constant<int, 4>());
            stp(s2, 2, corr);
            put(cur, nxt, s2, std::integral_constant<int, 5>());
            stp(s2, 3, corr);
            put(cur, nxt, s2, std::integral_constant<int, 6>());
            stp(s2, 4, corr);
            put(cur, nxt, s2, std::integral_constant<int, 7>());
            stp(s2, 5, corr);
            put(cur, nxt, s2, std::integral_constant<int, 8>());
            stp(s2, 6, corr);
            put(cur, nxt, s2, std::integral_constant<int, 9>());
            stp(s2, 7, corr);
        };
        put(cur, nxt, 0, std::integral_constant<int, 0>());
        for (int s2 = 0; s2 < slabs_per_task; ++s2) {
            if constexpr (kFlagged<Step>) {
                if (slab_flag(cg * slabs_per_task + s2)) {
                    slab_body(s2, std::true_type());
                } else {
                    slab_body(s2, std::false_type());
                }
            } else {
                slab_body(s2, std::false_type());
            }
        }
        // the two surplus indices of the task
        put(cur, nxt, slabs_per_task, std::integral_constant<int, 1>());
        put(cur, nxt, slabs_per_task, std::integral_constant<int, 2>());
        task_end(wave + q * NW);
    }
}

}  // namespace q4k

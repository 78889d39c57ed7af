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

namespace q4k {

constexpr int kRingRow = 2 * 128 + 16;        // two lines per row, padded
constexpr int kRingWave = 16 * kRingRow;

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
// (rr: the ring row of the lane's tile row j, b0: the superblock's byte
// offset in that row's two-line ring window, mod 256) and task_end(task)
// after each task's last slab.
template <int NW, int P, typename IssueX, typename ConvertX, typename Step, typename TaskEnd>
__device__ __forceinline__ void line_stream(const uint8_t* __restrict__ w,
                                            const float* __restrict__ x, int n, int S,
                                            int rows_per_block, int slabs_per_task,
                                            unsigned char* ring, IssueX issue_x,
                                            ConvertX convert_x, Step step, TaskEnd task_end)
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
    auto slab_of = [&](int sig, int& tile, int& slab) {
        sig = max(0, min(sig, my_slabs - 1));
        const int task = min(wave + (sig / slabs_per_task) * NW, ntasks - 1);
        tile = task / ncg;
        slab = (task % ncg) * slabs_per_task + sig % slabs_per_task;
    };
    // the two global addresses (rows lrow and 8 + lrow) of line l of slab
    // sig; past the wave's last slab the prefetch reads a 128-byte line of x
    // instead (cached, so the surplus loads cost no HBM traffic; each wave
    // takes its own line, or the tails of all waves would queue on one L2
    // channel).  The choice is a mask on the byte offset from w: a select of
    // two pointers makes the compiler branch around the address arithmetic,
    // which costs registers across the unrolled slab.
    const int xlines = S * 8;                        // 128-byte lines of one x vector
    const uint64_t dx = (uint64_t)(reinterpret_cast<const uint8_t*>(x) - w) +
                        (uint64_t)((blockIdx.x * NW + wave) % xlines) * 128u;
    auto line_ptrs = [&](int sig, int l, const uint8_t** p) {
        int tile, slab;
        slab_of(sig, tile, slab);
        const uint64_t mask = sig >= my_slabs ? ~0ull : 0ull;     // wave-uniform
        const uint64_t off = (uint64_t)(9 * slab + l) * 128;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = min(tile * 16 + 8 * h + lrow, rows_here - 1);
            const uint64_t full = (uint64_t)(row0 + r) * row_bytes + off;
            p[h] = w + (((full & ~mask) | (dx & mask)) + 16 * lunit);
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
#pragma unroll
    for (int l = 0; l < P; ++l) {
        const uint8_t* p[2];
        line_ptrs(0, l, p);
        lines[l][0] = load_line_nt(p[0]);
        lines[l][1] = load_line_nt(p[1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    convert_x();
    __syncthreads();

    for (int sig = 0; sig < my_slabs; ++sig) {
        int tile, slab;
        slab_of(sig, tile, slab);
        const uint32_t par = (uint32_t)slab & 1u;      // parity of line 9*slab
#pragma unroll
        for (int cp = 0; cp < 8; ++cp) {
            // lines written before superblock cp: 0 and 1 first, then cp + 1
#pragma unroll
            for (int l = (cp == 0 ? 0 : cp + 1); l <= cp + 1; ++l) {
                const int slot = l % P;
                const uint32_t lpos = ((par + (uint32_t)l) & 1u) * 128u + 16u * (uint32_t)lunit;
                *reinterpret_cast<uint4*>(ring + lrow * kRingRow + lpos) = lines[slot][0];
                *reinterpret_cast<uint4*>(ring + (8 + lrow) * kRingRow + lpos) = lines[slot][1];
                // memory operations stay in order here (the refill after the
                // write of its slot); arithmetic may move across
                __builtin_amdgcn_sched_barrier(0x000F);
                const int ln = l + P;              // refill: P lines ahead
                const uint8_t* p[2];
                line_ptrs(ln >= 9 ? sig + 1 : sig, ln >= 9 ? ln - 9 : ln, p);
                lines[slot][0] = load_line_nt(p[0]);
                lines[slot][1] = load_line_nt(p[1]);
            }
            // superblock c = 8 slab + cp, in the ring of tile row j
            step(8 * slab + cp, ring + j * kRingRow, (uint32_t)(144 * cp) + par * 128u);
        }
        if (sig % slabs_per_task == slabs_per_task - 1) {
            task_end(wave + (sig / slabs_per_task) * NW);
        }
    }
}

}  // namespace q4k

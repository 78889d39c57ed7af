"""CPU model of the index arithmetic of the line stream for rows of partial
slabs (`line_stream_any` in csrc/q4k_lines.h) and of the vector-ALU kernel's
ring addressing (`gemv_dot4_lines_kernel<..., true>` in csrc/q4k_dpp.hip).

The model replays, for every workgroup and wave, the stream's line loads
(which 16-byte piece of which row, or the wave's line of x), its ring writes
and register-slot refills, and every superblock step, and checks that

* each 16-byte piece a step reads from the ring is the weight piece of that
  row, superblock and task (so the schedule writes every line before a step
  needs it and never overwrites one a step still needs), and
* every weight load lies inside the matrix (16-byte aligned, below n * row
  bytes), i.e. no load runs past the last row.

It is a model written from the same design as the kernel, not the kernel:
the GPU parity tests check the kernel itself on the same kinds of shapes.
"""
import pytest


def simulate(n, S, NW, rpb, spt, P=3):
    RB = S * 144
    nslabs = (S + 7) // 8
    assert nslabs % spt == 0
    ncg = nslabs // spt
    lpt = 9 * spt + 3
    grid = (n + rpb - 1) // rpb
    w_end = n * RB
    steps = 0
    for blk in range(grid):
        row0 = blk * rpb
        rows_here = min(rpb, n - row0)
        ntiles = (rows_here + 15) // 16
        ntasks = ntiles * ncg
        for wave in range(NW):
            my_tasks = (ntasks - wave + NW - 1) // NW if ntasks > wave else 0

            def task_of(q):
                qc = max(0, min(q, my_tasks - 1))
                task = min(wave + qc * NW, ntasks - 1)
                tile, cg = task // ncg, task % ncg
                return tile, cg, min(8 * spt, S - 8 * cg * spt)

            def load(q, L):
                tile, cg, T = task_of(q)
                past = q >= my_tasks
                out = {}
                for rr in range(16):                 # ring rows = loader rows
                    r = min(tile * 16 + rr, rows_here - 1)
                    start = (row0 + r) * RB
                    off = start & 127
                    for lu in range(8):
                        piece = 128 * L + 16 * lu
                        if (not past) and piece < off + 144 * T:
                            addr = start - off + cg * spt * 1152 + piece
                            assert 0 <= addr and addr + 16 <= w_end and addr % 16 == 0
                            out[(rr, lu)] = addr
                        else:
                            out[(rr, lu)] = None     # the wave's line of x
                return out

            slots = [load(0, l) for l in range(P)]
            ring = {}

            def put(q, s2, X):
                slot = X % P
                L = 9 * s2 + X
                for (rr, lu), v in slots[slot].items():
                    ring[(rr, L & 3, lu)] = v
                ln = L + P
                slots[slot] = load(q + 1, ln - lpt) if ln >= lpt else load(q, ln)

            def step(q, c, b0):
                tile, _, _ = task_of(q)
                for j in range(16):
                    if tile * 16 + j >= rows_here:
                        continue                     # row past n: result discarded
                    loff = (j * 144 * S) & 127
                    start = (row0 + tile * 16 + j) * RB
                    assert start & 127 == loff       # tiles start on a line
                    for g in range(4):
                        for rel in (0, 16 + 32 * g, 32 + 32 * g):
                            pos = (b0 + loff + rel) & 511
                            got = ring[(j, pos >> 7, (pos & 127) // 16)]
                            assert got == start + c * 144 + rel, (blk, wave, q, c, j, g, rel)

            for q in range(my_tasks):
                _, cg, T = task_of(q)
                c0 = 8 * cg * spt
                put(q, 0, 0)
                for s2 in range(spt):
                    # lines 9 s2 + X written before superblock cp of the slab
                    for X, cp in ((1, 0), (2, None), (3, 1), (4, 2), (5, 3), (6, 4), (7, 5),
                                  (8, 6), (9, 7)):
                        put(q, s2, X)
                        if cp is not None and 8 * s2 + cp < T:
                            step(q, c0 + 8 * s2 + cp, 1152 * s2 + 144 * cp)
                            steps += 1
                put(q, spt, 1)
                put(q, spt, 2)
    return steps


SHAPES = [(4096, 43), (17, 5), (130, 20), (33, 54), (1, 1), (16, 3), (300, 13), (257, 9),
          (64, 7), (40, 17)]


@pytest.mark.parametrize("n,S", SHAPES)
def test_line_stream_any_model(n, S):
    nslabs = (S + 7) // 8
    ntiles = (n + 15) // 16
    for NW in (4, 8, 16):
        for rpb in sorted({16 * ((ntiles + 255) // 256), 48, 16, 80}):
            for spt in sorted({1, nslabs}):
                if n > 1000 and (NW != 8 or rpb != 16):
                    continue
                steps = simulate(n, S, NW, rpb, spt)
                # every superblock column of every 16-row tile, once
                tiles = sum((min(rpb, n - b) + 15) // 16 for b in range(0, n, rpb))
                assert steps == tiles * S


def lookahead_columns(n, S, NW, rpb, spt, kA, aligned):
    """Replay kernel 6's per-wave x look-ahead (gemv_i8_sub_kernel<..., true,
    ANY> in csrc/q4k_mfma.hip) over the columns the streams step through:
    register slot cp % kA must hold column c whenever step (c, cp) is
    valid.  The streams pass cend (end of the slab's or task's columns) and
    cn (first column of the wave's next slab or task, clamped to its last)."""
    nslabs = (S + 7) // 8
    ncg = nslabs // spt
    grid = (n + rpb - 1) // rpb
    checked = 0
    for blk in range(grid):
        rows_here = min(rpb, n - blk * rpb)
        ntasks = ((rows_here + 15) // 16) * ncg
        for wave in range(NW):
            my_tasks = (ntasks - wave + NW - 1) // NW if ntasks > wave else 0
            # steps as the stream issues them: (c, cend, cn, cp, valid)
            seq = []
            if aligned:
                my_slabs = my_tasks * spt

                def slab_of(sig):
                    sig = max(0, min(sig, my_slabs - 1))
                    task = min(wave + (sig // spt) * NW, ntasks - 1)
                    return (task % ncg) * spt + sig % spt
                for sig in range(my_slabs):
                    slab, slab_n = slab_of(sig), slab_of(sig + 1)
                    for cp in range(8):
                        seq.append((8 * slab + cp, 8 * slab + 8, 8 * slab_n, cp, True))
            else:
                def task_of(q):
                    qc = max(0, min(q, my_tasks - 1))
                    task = min(wave + qc * NW, ntasks - 1)
                    cg = task % ncg
                    return cg, min(8 * spt, S - 8 * cg * spt)
                for q in range(my_tasks):
                    cg, T = task_of(q)
                    cg_n, _ = task_of(q + 1)
                    c0, cn = 8 * cg * spt, 8 * cg_n * spt
                    for s2 in range(spt):
                        for cp in range(8):
                            seq.append((c0 + 8 * s2 + cp, c0 + 8 * spt, cn, cp, 8 * s2 + cp < T))
            # the kernel: prologue loads columns c_first + a into slot a
            task0 = min(wave, ntasks - 1) if ntasks else 0
            c_first = 8 * ((task0 % ncg) * spt) if ntasks else 0
            slots = {a: c_first + a for a in range(kA)}
            for c, cend, cn, cp, valid in seq:
                if valid:
                    assert slots[cp % kA] == c, (blk, wave, c, slots)
                    assert 0 <= c < S
                    checked += 1
                ca = c + kA if c + kA < cend else cn + (c + kA - cend)
                slots[cp % kA] = min(ca, S - 1)      # loads clamp to the last column
    return checked


@pytest.mark.parametrize("n,S,spt,aligned", [
    (4096, 56, 1, True), (130, 16, 2, True), (300, 32, 1, True), (48, 112, 2, True),
    (4096, 43, 1, False), (130, 5, 1, False), (257, 20, 3, False), (17, 54, 1, False),
    (300, 13, 2, False), (1, 1, 1, False),
])
@pytest.mark.parametrize("kA", [2, 4])
def test_jit_lookahead_columns(n, S, spt, aligned, kA):
    nslabs = (S + 7) // 8
    if nslabs % spt:
        pytest.skip("column groups must divide the slabs")
    for rpb in (16, 48, 128):
        checked = lookahead_columns(n, S, 8, rpb, spt, kA, aligned)
        assert checked == ((n + 15) // 16) * S      # every tile's columns, once each

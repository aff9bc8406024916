"""Host model of the GEMM's output stores (no GPU).

Lane (q, fr) of a wave holds, for m-block mb and n-block nb, output row 16 mb + fr
at the 4 columns colB(nb) .. +3, colB(nb) = 32 (nb // 2) + 4 (nb % 2) + 8q.  The
kernel's full-tile stores trade 16 bytes between lanes fr and fr ^ 1 (a DPP
quad_perm [1,0,3,2] swap) so that every store instruction covers whole 128-byte
row segments.  This model replays the lane arithmetic of the bf16 and fp32 stores as
the kernel source writes it, with each value labelled by its (row, column), and
checks that every output of the wave's 64 x (16 nb) tile is stored exactly once, at
its own place, and that each store instruction writes complete 128-byte segments.
"""
import pytest


def col_b(nb, q):
    return 32 * (nb >> 1) + 4 * (nb & 1) + 8 * q


def lane_values(mb, nb, q, fr):
    """The (row, column) labels of acc[mb][nb] in lane (q, fr)."""
    return [(16 * mb + fr, col_b(nb, q) + e) for e in range(4)]


def swap(values_by_lane):
    return {(q, fr): values_by_lane[(q, fr ^ 1)] for (q, fr) in values_by_lane}


def bf16_stores(nblocks, width):
    """Per store instruction: lane -> (row, first column, 8 labelled values).  Addresses are
    kept as (row, column) pairs of the wave's tile; `width` is the row pitch in elements."""
    instrs = []
    for mb in range(4):
        for t in range(nblocks // 4):
            d0, d1 = {}, {}
            for q in range(4):
                for fr in range(16):
                    d0[(q, fr)] = lane_values(mb, 4 * t, q, fr) + lane_values(mb, 4 * t + 1, q, fr)
                    d1[(q, fr)] = lane_values(mb, 4 * t + 2, q, fr) + lane_values(mb, 4 * t + 3, q, fr)
            e = {k: (d0[k] if k[1] & 1 else d1[k]) for k in d0}
            sw = swap(e)
            x, y = {}, {}
            for (q, fr) in d0:
                odd = fr & 1
                cx = 8 * (q + 4 * (fr & 1))
                x[(q, fr)] = (16 * mb + (fr & ~1), cx + 64 * t, sw[(q, fr)] if odd else d0[(q, fr)])
                y[(q, fr)] = (16 * mb + (fr | 1), cx + 64 * t, d1[(q, fr)] if odd else sw[(q, fr)])
            instrs += [x, y]
    return instrs, 2


def f32_stores(nblocks, width):
    instrs = []
    for mb in range(4):
        for pp in range(nblocks // 2):
            a0, a1 = {}, {}
            for q in range(4):
                for fr in range(16):
                    a0[(q, fr)] = lane_values(mb, 2 * pp, q, fr)
                    a1[(q, fr)] = lane_values(mb, 2 * pp + 1, q, fr)
            e = {k: (a0[k] if k[1] & 1 else a1[k]) for k in a0}
            sw = swap(e)
            x, y = {}, {}
            for (q, fr) in a0:
                odd = fr & 1
                cx = 8 * q + 4 * (fr & 1)
                x[(q, fr)] = (16 * mb + (fr & ~1), 32 * pp + cx, sw[(q, fr)] if odd else a0[(q, fr)])
                y[(q, fr)] = (16 * mb + (fr | 1), 32 * pp + cx, a1[(q, fr)] if odd else sw[(q, fr)])
            instrs += [x, y]
    return instrs, 4


@pytest.mark.parametrize("kind", ["bf16", "fp32"])
@pytest.mark.parametrize("nblocks", [8, 4])
def test_every_output_stored_once_in_whole_segments(kind, nblocks):
    width = 16 * nblocks
    instrs, esize = (bf16_stores if kind == "bf16" else f32_stores)(nblocks, width)
    seen = {}
    for instr in instrs:
        segments = {}
        for (row, col, vals) in instr.values():
            for i, label in enumerate(vals):
                assert label == (row, col + i), (kind, row, col, i, label)
                seen[label] = seen.get(label, 0) + 1
                byte = (row * width + col + i) * esize
                segments.setdefault(byte // 128, set()).add(byte % 128)
        # each instruction covers complete 128-byte segments of the output rows
        for seg, offsets in segments.items():
            assert offsets == set(range(0, 128, esize)), (kind, seg, sorted(offsets))
    assert len(seen) == 64 * width and set(seen.values()) == {1}

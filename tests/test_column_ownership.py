"""Column ownership of float4 lanes at widths that are not a multiple of 4
(host model of the kernels' lane-to-column map, no GPU).

Lane g of a row's group, coarsening step f, in the column slice starting at
c0 owns the vector starting at c = c0 + (f*G + g)*VEC while c < c_end; the
vector that would run past c_end is moved back to start at c_end - VEC and
stores only its elements past (c - (c_end - VEC)).  These tests enumerate
launch shapes and check the two properties the kernels rely on: every read
stays inside [c_begin_of_row = 0, N) and every column of [c_begin, c_end) is
written by exactly one lane.  The split's column passes are checked the same
way: a last pass narrower than one vector starts earlier, and each pass
stays at least one vector wide.
"""
import itertools

import pytest

PARTIAL_WIDTH = 256   # columns per pass of the split path


def lanes(c_begin, c_end, G, F, VEC):
    """(first column read, first element stored) per owning lane."""
    SL = G * F * VEC
    slices = (c_end - c_begin + SL - 1) // SL
    out = []
    for s in range(slices):
        c0 = c_begin + s * SL
        for f, g in itertools.product(range(F), range(G)):
            c = c0 + (f * G + g) * VEC
            if c >= c_end:
                continue
            colf = c_end - VEC if (VEC > 1 and c > c_end - VEC) else c
            cc = colf - c_begin
            skip = (VEC - (cc & (VEC - 1))) & (VEC - 1)
            out.append((colf, skip))
    return out


@pytest.mark.parametrize("VEC", [1, 2, 4])
def test_each_column_written_once_and_reads_in_row(VEC):
    for N in list(range(VEC, 70)) + [129, 130, 131, 257, 258, 259, 513, 602, 1433]:
        for G, F in itertools.product((4, 8, 16, 32, 64), (1, 2)):
            if VEC == 2 and N % 2:
                continue   # float2 lanes need an even width
            written = [0] * N
            for colf, skip in lanes(0, N, G, F, VEC):
                assert 0 <= colf and colf + VEC <= N, (N, G, F, VEC, colf)
                for e in range(skip, VEC):
                    written[colf + e] += 1
            assert written == [1] * N, (N, G, F, VEC)


def test_split_passes():
    for N in list(range(4, 40)) + [255, 256, 257, 258, 259, 260, 511, 512, 513, 514, 515, 1433]:
        vec = 4
        covered = [0] * N
        for p0 in range(0, N, PARTIAL_WIDTH):
            w1 = min(N, p0 + PARTIAL_WIDTH)
            w0 = min(p0, max(0, w1 - vec))          # as in the library's pass loop
            assert 0 <= w0 and w1 - w0 >= vec and w1 - w0 <= PARTIAL_WIDTH, (N, p0)
            for colf, skip in lanes(w0, w1, 64, 1, vec):
                assert w0 <= colf and colf + vec <= w1
                for e in range(skip, vec):
                    covered[colf + e] += 1
        # a narrow last pass recomputes up to 3 columns of the previous pass
        # (sequential launches, same bits): every column at least once
        assert min(covered) >= 1 and max(covered) <= 2, N

"""CPU simulation of the 16x16-form tiled kernel's LDS indexing (k_tiled16 in
csrc/kernels_k16.hip) for both wave arrangements.

One K tile of A (256 rows) and B (256 rows) is 64 bytes per row, stored in
LDS as 16-byte chunks: chunk c of row r at row * 64 + 16 (c ^ swz16(r)), with
swz16(r) = (r >> 1) & 3 (chosen by measuring bank conflicts of this read
pattern on the hardware).  512 threads copy it: thread t owns chunk t % 4 of
rows t / 4 + 128 i (W4A16: threads 2c and 2c + 1 write chunks 0-1 and 2-3 of
B row c).  A fragment read by lane l of block b takes row base + 16 b +
l % 16, chunk l / 16.  The simulation checks that the copy writes every byte
of the stage exactly once and inside it, that every fragment read returns the
bytes of the row and K range it stands for, that A and B fragments of one
MFMA pair equal K, and that every output of a wave's block is covered exactly
once by one (A block, B block) pair."""
import pytest

BKB, NT, CH = 64, 512, 4
RPP = NT // CH


def swz16(r):
    return (r >> 1) & 3


def slot(r, c):
    return r * BKB + 16 * (c ^ swz16(r))


@pytest.mark.parametrize("GM,GN", [(2, 4), (4, 2)], ids=["tiled256w8k16", "tiled256w8tk16"])
def test_k16_lds_indexing(GM, GN):
    BM = BN = 256
    A_TILE = BM * BKB
    stage = {}
    for t in range(NT):
        ch, r0 = t % CH, t // CH
        for op, base, rows in (("A", 0, BM), ("B", A_TILE, BN)):
            for i in range(rows // RPP):
                r = r0 + i * RPP
                off = base + slot(r0, ch) + i * RPP * BKB  # the kernel's l0 + i RPP BKB
                assert off == base + slot(r, ch)           # swz16 is RPP-periodic
                for b in range(16):
                    assert off + b not in stage
                    stage[off + b] = (op, r, 16 * ch + b)
    assert len(stage) == (BM + BN) * BKB and max(stage) < (BM + BN) * BKB

    WM, WN = BM // GM, BN // GN
    FI, FJ = WM // 16, WN // 16
    for wave in range(GM * GN):
        wm, wn = wave // GN, wave % GN
        covered = set()
        for lane in range(64):
            arow = wm * WM + (lane & 15)
            brow = wn * WN + (lane & 15)
            grp = lane >> 4
            a_off = arow * BKB + 16 * (grp ^ swz16(arow))
            b_off = A_TILE + brow * BKB + 16 * (grp ^ swz16(brow))
            for i in range(FI):
                got = [stage[a_off + i * 16 * BKB + q] for q in range(16)]
                assert got == [("A", arow + 16 * i, 16 * grp + q) for q in range(16)]
            for j in range(FJ):
                got = [stage[b_off + j * 16 * BKB + q] for q in range(16)]
                assert got == [("B", brow + 16 * j, 16 * grp + q) for q in range(16)]
            # accumulator register r of (i, j): row 4 (l / 16) + r, column l % 16
            for i in range(FI):
                for j in range(FJ):
                    for r in range(4):
                        out = (wm * WM + 16 * i + 4 * (lane >> 4) + r, wn * WN + 16 * j + lane % 16)
                        assert out not in covered
                        covered.add(out)
        assert len(covered) == WM * WN


def test_k16_w4_b_rows():
    """W4A16: threads 2c, 2c + 1 write chunks 2h, 2h + 1 of B row c, i.e. K
    16h .. 16h + 15 of the tile; every slot of the B tile written once."""
    seen = set()
    for t in range(NT):
        col, half = t >> 1, t & 1
        for q in range(2):
            off = col * BKB + 16 * ((2 * half + q) ^ swz16(col))
            assert off == slot(col, 2 * half + q)
            assert off not in seen
            seen.add(off)
    assert len(seen) == 256 * 4

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


def swz64(r):
    return (r >> 2) & 3


@pytest.mark.parametrize("GM,GN,FB", [(2, 4, 16), (4, 2, 16), (2, 4, 32), (4, 2, 32)],
                         ids=["tiled256w8k16", "tiled256w8tk16", "fp8_2x4", "fp8_4x2"])
def test_k16_lds_indexing(GM, GN, FB):
    """FB = 16: 16x16 fragments, one 16-byte read per lane at chunk l / 16,
    slot function swz16.  FB = 32 (fp8, 32x32x64): two reads per lane at
    chunks 2 (l / 32) and 2 (l / 32) + 1, slot function swz64."""
    sw = swz16 if FB == 16 else swz64
    NRD = 1 if FB == 16 else 2

    def slot(r, c):
        return r * BKB + 16 * (c ^ sw(r))

    BM = BN = 256
    A_TILE = BM * BKB
    stage = {}
    for t in range(NT):
        ch, r0 = t % CH, t // CH
        for op, base, rows in (("A", 0, BM), ("B", A_TILE, BN)):
            for i in range(rows // RPP):
                r = r0 + i * RPP
                off = base + slot(r0, ch) + i * RPP * BKB  # the kernel's l0 + i RPP BKB
                assert off == base + slot(r, ch)           # the slot function is RPP-periodic
                for b in range(16):
                    assert off + b not in stage
                    stage[off + b] = (op, r, 16 * ch + b)
    assert len(stage) == (BM + BN) * BKB and max(stage) < (BM + BN) * BKB

    WM, WN = BM // GM, BN // GN
    FI, FJ = WM // FB, WN // FB
    for wave in range(GM * GN):
        wm, wn = wave // GN, wave % GN
        covered = set()
        for lane in range(64):
            arow = wm * WM + (lane & (FB - 1))
            brow = wn * WN + (lane & (FB - 1))
            grp = lane >> 4 if FB == 16 else 2 * (lane >> 5)
            for q in range(NRD):
                a_off = arow * BKB + 16 * ((grp + q) ^ sw(arow))
                b_off = A_TILE + brow * BKB + 16 * ((grp + q) ^ sw(brow))
                for i in range(FI):
                    got = [stage[a_off + i * FB * BKB + e] for e in range(16)]
                    assert got == [("A", arow + FB * i, 16 * (grp + q) + e) for e in range(16)]
                for j in range(FJ):
                    got = [stage[b_off + j * FB * BKB + e] for e in range(16)]
                    assert got == [("B", brow + FB * j, 16 * (grp + q) + e) for e in range(16)]
            # accumulator register r of block (i, j): 16x16: row 4 (l / 16) + r,
            # column l % 16; 32x32: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
            for i in range(FI):
                for j in range(FJ):
                    for r in range(4 if FB == 16 else 16):
                        if FB == 16:
                            rr, cc = 4 * (lane >> 4) + r, lane % 16
                        else:
                            rr, cc = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), lane % 32
                        out = (wm * WM + FB * i + rr, wn * WN + FB * j + cc)
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

"""CPU simulation of the 16x16-form tiled kernel's LDS indexing (k_tiled16 in
csrc/kernels_k16.hip) for both wave arrangements.

One K tile of A (256 rows) and B (256 rows) is 64 bytes per row, stored in
LDS as 16-byte chunks: chunk c of row r at row * 64 + 16 (c ^ swz64(r)), with
swz64(r) = (r >> 2) & 3.  512 threads copy it: thread t owns chunk t % 4 of
rows t / 4 + 128 i.  A fragment read by lane l of block b takes row
base + 16 b + l % 16, chunk l / 16.  The simulation checks that the copy
writes every byte of the stage exactly once and inside it, that every
fragment read returns the bytes of the row and K range it stands for, that A
and B fragments of one MFMA pair equal K, that every output of a wave's
block is covered exactly once by one (A block, B block) pair, and that the
16 lanes of a read group hit 16 distinct 16-byte slots of a 256-byte bank
window (no bank conflict)."""
import pytest

BKB, NT, CH = 64, 512, 4
RPP = NT // CH


def swz64(r):
    return (r >> 2) & 3


def slot(r, c):
    return r * BKB + 16 * (c ^ swz64(r))


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
                assert off == base + slot(r, ch)           # swz64 is RPP-periodic
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
            a_off = arow * BKB + 16 * (grp ^ swz64(arow))
            b_off = A_TILE + brow * BKB + 16 * (grp ^ swz64(brow))
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
        # bank check: lanes 16 g .. 16 g + 15 of one fragment read
        for grp in range(4):
            for base_row in (wm * WM, wn * WN):
                addrs = [slot(base_row + l, grp) % 256 for l in range(16)]
                assert len(set(addrs)) == 16

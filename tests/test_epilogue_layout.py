"""CPU simulation of the LDS-staged epilogue's indexing (epilogue_slabs in
csrc/device_common.hpp) for every wave tile the kernels instantiate.

Per 32-row slab, each lane writes its accumulator registers to LDS (register
r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of a
32x32 fragment; fragment j of the slab sits at column 32 j; on the 16x16
forms register r of lane l holds row 4 (l / 16) + r, column l % 16 of a 16x16
fragment, and a slab holds fragment rows 2 i and 2 i + 1), then reads back
four consecutive columns of one row per pass.  The simulation replays both
index formulas and checks that the writes are a bijection onto the slab's
words, that each pass reads exactly the words written for the outputs it
stores (the value read for output (row, col) is the one written for it),
that every word lies inside the wave's own region, that the regions of a
workgroup's waves are disjoint and inside the kernel's LDS allocation, and
that the row handled by each lane in each pass is the one whose C and D
offsets it uses.  Integer and float accumulators use the same indexing
(integers are converted to fp32 as they are written, before the slab
barrier), so the integer -> float epilogue needs no other layout."""
import pytest

# (name, waves, wave tile WM x WN, LDS bytes the K loop needs, fragment size)
KERNELS = [
    ("tiled256 (4 waves)", 4, 128, 128, 3 * 2 * 256 * 64, 32),
    ("tiled256w8", 8, 128, 64, 3 * 2 * 256 * 64, 32),
    ("tiled256w8t", 8, 64, 128, 3 * 2 * 256 * 64, 32),
    ("tiled256w8k16", 8, 128, 64, 3 * 2 * 256 * 64, 16),
    ("tiled256w8tk16", 8, 64, 128, 3 * 2 * 256 * 64, 16),
    ("tiled128", 4, 64, 64, 3 * 2 * 128 * 64, 32),
    ("sparse24_dma8", 8, 128, 64, 3 * (256 * 64 + 256 * 128) + 2 * 256 * 32, 32),
    ("sparse24_tiled", 4, 128, 128, 2 * (256 * 64 + 256 * 16 + 256 * 128), 32),
]


def staged(i, FN, FB, lane):
    """(slab row, slab column, register id) of every accumulator value lane
    `lane` writes for slab i (FB = 32 or 16 fragment rows / columns)."""
    out = []
    if FB == 32:
        for j in range(FN):
            for r in range(16):
                out.append((8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), j * 32 + (lane & 31),
                            (i, j, r)))
    else:
        for h in range(2):
            for j in range(FN):
                for r in range(4):
                    out.append((16 * h + 4 * (lane >> 4) + r, j * 16 + (lane & 15),
                                (2 * i + h, j, r)))
    return out


def simulate(WM, WN, FB):
    FM, FN = WM // FB, WN // FB
    COLS, PITCH = FB * FN, FB * FN + 4
    LPR = COLS // 4
    RPP = 64 // LPR
    NP = 32 // RPP
    assert LPR * RPP == 64 and NP * RPP == 32
    regs = set()
    for i in range(FM * FB // 32):  # one slab per 32 rows
        written = {}
        for lane in range(64):
            for row, col, reg in staged(i, FN, FB, lane):
                # register reg of lane `lane` is output (FB fi + row % FB ...):
                # the fragment's own layout, checked against the slab position
                fi, fj, r = reg
                if FB == 32:
                    assert (fi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), fj * 32 + lane % 32) \
                        == (32 * i + row, col)
                else:
                    assert (fi * 16 + 4 * (lane >> 4) + r, fj * 16 + lane % 16) == (32 * i + row, col)
                regs.add((reg, lane))
                w = row * PITCH + col
                assert 0 <= w < 32 * PITCH
                assert w not in written, (i, reg, lane)
                written[w] = (32 * i + row, col)
        assert len(written) == 32 * COLS
        seen = set()
        for p in range(NP):
            for lane in range(64):
                rl, c4 = lane // LPR, (lane % LPR) * 4
                rr = p * RPP + rl
                for q in range(4):
                    w = rr * PITCH + c4 + q
                    out = (32 * i + rr, c4 + q)
                    assert written[w] == out, (i, p, lane, q)
                    assert out not in seen
                    seen.add(out)
                # the C / D offsets of this lane and pass: row rl + p RPP of
                # the slab (vd = rl * ldd + col, soff = (32 i + p RPP) * ldd)
                assert rr == rl + p * RPP
        assert len(seen) == 32 * COLS
    # every accumulator register of every lane is staged exactly once
    assert len(regs) == WM * WN
    return 32 * PITCH * 4  # bytes per wave


@pytest.mark.parametrize("name,waves,WM,WN,kloop,FB", KERNELS, ids=[k[0] for k in KERNELS])
def test_epilogue_slab_indexing(name, waves, WM, WN, kloop, FB):
    per_wave = simulate(WM, WN, FB)
    # waves w own [w * per_wave, (w + 1) * per_wave): disjoint by construction;
    # the kernel's allocation is max(K loop, epilogue)
    total = waves * per_wave
    assert total == waves * 32 * (WN + 4) * 4
    assert max(kloop, total) <= 160 * 1024

"""The kernels' LDS layouts under the gfx950 bank model (host only).

Model (measured with hgemm_probe_lds_read: a lane-contiguous 16-byte read
runs at ~240 bytes/clock/CU): 64 banks of 4 bytes; a 16-byte-per-lane access
is served 16 lanes at a time, and two lanes of one group whose addresses fall
on the same bank (different 256-byte lines) conflict.

Access patterns of the register-staged baseline kernel (its four LDS
layouts):
  write: thread t stores chunk t % 8 of row t // 8 (+ multiples of 32 rows),
  read:  lane l of a wave reads logical chunk 2*ks + l // 32 of row l % 32
         of a 32-row fragment (ks = 0..3).
The production kernels' placement (direct-to-LDS segments, 16-byte and
transposing fragment reads) is checked at the end of the file.
"""
import numpy as np
import pytest

from dense_half_precision_amd import hgemm


def conflicts(addrs):
    """Extra cycles of one 16-lane group: max lanes sharing a bank, minus 1."""
    banks = {}
    for a in addrs:
        for w in range(4):
            b = ((a + 4 * w) // 4) % 64
            banks.setdefault(b, set()).add((a + 4 * w) // 256)
    return max(len(v) for v in banks.values()) - 1


def read_groups(off, row0=0):
    for ks in range(4):
        lanes = [off[row0 + (l % 32)][2 * ks + l // 32] for l in range(64)]
        for g in range(4):
            yield lanes[16 * g:16 * g + 16]


def write_groups(off):
    for t0 in range(0, 256, 16):
        yield [off[t // 8][t % 8] for t in range(t0, t0 + 16)]


@pytest.mark.parametrize("layout", [hgemm.LDS_XOR, hgemm.LDS_PLAIN, hgemm.LDS_PAD,
                                    hgemm.LDS_XOR_ROW])
def test_layout_is_a_bijection_per_row(layout):
    off = hgemm.lds_offsets(layout)
    rowb = 144 if layout == hgemm.LDS_PAD else 128
    for r, row in enumerate(off):
        assert sorted(row) == [r * rowb + 16 * c for c in range(8)]


# (layout, extra cycles of the worst read group, of the worst write group):
# only the row/2 XOR swizzle is conflict-free both ways; padding to 144 bytes
# fixes the reads but makes row 1's last chunk wrap onto row 0's first banks.
@pytest.mark.parametrize("layout,read_conf,write_conf", [
    (hgemm.LDS_XOR, 0, 0), (hgemm.LDS_PAD, 0, 1), (hgemm.LDS_XOR_ROW, 1, 0),
    (hgemm.LDS_PLAIN, 7, 0)])
def test_bank_conflicts(layout, read_conf, write_conf):
    off = hgemm.lds_offsets(layout)
    worst_read = max(conflicts(g) for r0 in (0, 32, 64, 224) for g in read_groups(off, r0))
    worst_write = max(conflicts(g) for g in write_groups(off))
    assert worst_read == read_conf
    assert worst_write == write_conf


# ---------------------------------------------------------------- production
@pytest.mark.parametrize("mn_major", [0, 1])
@pytest.mark.parametrize("bx", [64, 128, 256])
def test_production_operand_placement(mn_major, bx):
    """The production kernels' direct-to-LDS placement and fragment reads
    (the functions the kernels use, run on the host): every chunk of the tile
    is loaded exactly once, every fragment read points at the data the matrix
    core operand needs (8 consecutive k of one row/column per lane), and the
    reads are free of bank conflicts under the 64-bank model (16-byte reads
    served 16 lanes at a time, 8-byte reads 32 at a time)."""
    lr, lc, ro = hgemm.operand_offsets(mn_major, bx)
    rows, chunks = (64, bx // 8) if mn_major else (bx, 8)
    pairs = list(zip(lr.ravel().tolist(), lc.ravel().tolist()))
    assert len(set(pairs)) == len(pairs) == rows * chunks
    assert all(0 <= r < rows and 0 <= c < chunks for r, c in pairs)
    loc = {p: 1024 * (i // 64) + 16 * (i % 64) for i, p in enumerate(pairs)}
    lane = np.arange(64)
    for f in range(bx // 16):
        for sl in range(2):
            if not mn_major:
                want = [loc[(16 * f + l % 16, 4 * sl + l // 16)] for l in lane]
                assert ro[f, sl, 0].tolist() == want, (f, sl)
                for q in range(4):
                    o = ro[f, sl, 0, 16 * q:16 * q + 16]
                    banks = {(x // 4 + b) % 64 for x in o for b in range(4)}
                    assert len(banks) == 64, (f, sl, q)
            else:
                for h in range(2):
                    g, i = lane // 16, lane % 16
                    k = 32 * sl + 8 * g + i // 4 + 4 * h
                    col = 16 * f + 4 * (i % 4)
                    want = [loc[(int(kk), int(cc) // 8)] + (int(cc) % 8) * 2 for kk, cc in zip(k, col)]
                    assert ro[f, sl, h].tolist() == want, (f, sl, h)
                    for half in range(2):
                        o = ro[f, sl, h, 32 * half:32 * half + 32]
                        banks = {(x // 4 + b) % 64 for x in o for b in range(2)}
                        assert len(banks) == 64, (f, sl, h, half)


def test_ping_pong_slice_placement():
    """The two-group kernel's slice layout (the functions the kernel uses, run
    on the host): every (row, chunk) of a 256-row, 4-chunk slice is loaded
    exactly once; each fragment read points at row 16f + l%16, chunk l/16,
    the matrix-core operand; and the 16-lane groups of every read cover the
    64 banks once."""
    lr, lc, ro = hgemm.pp_offsets()
    pairs = list(zip(lr.ravel().tolist(), lc.ravel().tolist()))
    assert len(set(pairs)) == len(pairs) == 256 * 4
    assert all(0 <= r < 256 and 0 <= c < 4 for r, c in pairs)
    loc = {p: 1024 * (i // 64) + 16 * (i % 64) for i, p in enumerate(pairs)}
    lane = np.arange(64)
    for f in range(16):
        want = [loc[(16 * f + l % 16, l // 16)] for l in lane]
        assert ro[f].tolist() == want, f
        for q in range(4):
            o = ro[f, 16 * q:16 * q + 16]
            banks = {(x // 4 + b) % 64 for x in o for b in range(4)}
            assert len(banks) == 64, (f, q)


"""The kernels' LDS layouts under the gfx950 bank model (host only).

Model (measured with hgemm_probe_lds_read: a lane-contiguous 16-byte read
runs at ~240 bytes/clock/CU): 64 banks of 4 bytes; a 16-byte-per-lane access
is served 16 lanes at a time, and two lanes of one group whose addresses fall
on the same bank (different 256-byte lines) conflict.

Access patterns (from the kernel):
  write: thread t stores chunk t % 8 of row t // 8 (+ multiples of 32 rows),
  read:  lane l of a wave reads logical chunk 2*ks + l // 32 of row l % 32
         of a 32-row fragment (ks = 0..3).
"""
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

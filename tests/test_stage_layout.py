"""Host model of the LDS staging layout of the bf16 tile epilogue (gemm.hpp:
PairStageW writes, copy_staged reads), used by the down GEMM, the gate/up
data gradient and the MX and shared-expert down launches.

The epilogue stages a 256 x 256 bf16 tile in two 64 KiB stages (rows 0-127,
then 128-255).  Paired writers: lanes 2k, 2k+1 of a wave hold columns c, c+1 of
accumulator rows; for rows e, e+1 the even lane writes both columns of row e
and the odd lane both of row e+1 as one dword, at 16-byte chunk
q ^ (4 * swz(row)) of the row, swz(row) = (row & 1) | ((row >> 1) & 2).  The
reader takes chunk q of row r from chunk q ^ (4 * swz(r)).  These tests check,
for the two wave grids the kernels use (4 x 2 forward, 2 x 4 data-gradient),
that every element written is read back at its (row, column), that no two
writes overlap, and that the 64 lanes of one write instruction never hit the
same LDS bank twice (64 banks of 4 bytes, and 32 banks per half-wave).
"""
import pytest

STAGE = 65536


def swz(row):
    return (row & 1) | ((row >> 1) & 2)


def write_addr(nc, wm_count, wm, wn_base_col, lane, mi, e, c, off):
    odd, hi = lane & 1, lane >> 5
    r0 = wm * (256 // wm_count)
    base = (r0 >> 7) * STAGE + off + ((r0 & 127) + 4 * hi + odd) * nc * 2
    col = wn_base_col + (lane & 30) + c
    a = base + (mi * 32 + 8 * (e >> 2) + (e & 3)) * nc * 2 + (((col >> 3) ^ (4 * (odd | (hi << 1)))) << 4) + (col & 7) * 2
    row = r0 + 4 * hi + mi * 32 + 8 * (e >> 2) + (e & 3) + odd
    return a, row, col


@pytest.mark.parametrize("WM,WN", [(4, 2), (2, 4)])
def test_paired_staging_round_trip_and_banks(WM, WN):
    nc, off = 256, 0
    MI, nblk = 256 // WM // 32, 256 // WN // 32
    mem = {}
    for wave in range(WM * WN):
        wm, wn = wave // WN, wave % WN
        for mi in range(MI):
            for ni in range(nblk):
                for e in range(0, 16, 2):
                    addrs = []
                    for lane in range(64):
                        a, row, col = write_addr(nc, WM, wm, wn * nblk * 32, lane, mi, e, ni * 32, off)
                        assert a % 4 == 0
                        for k in range(2):
                            assert a + 2 * k not in mem
                            mem[a + 2 * k] = (row, col + k)
                        addrs.append(a // 4)
                    assert len(set(addrs)) == 64
                    assert len({d % 64 for d in addrs}) == 64
                    for h in (0, 32):
                        assert len({d % 32 for d in addrs[h:h + 32]}) == 32
    assert len(mem) == 256 * nc
    cpr = nc // 8
    for c in range(256 * cpr):
        row, q = c // cpr, c % cpr
        src = (row >> 7) * STAGE + off + (row & 127) * nc * 2 + ((q ^ (4 * swz(row))) << 4)
        for k in range(8):
            assert mem[src + 2 * k] == (row, q * 8 + k)
    assert min(mem) == 0 and max(mem) < 2 * STAGE  # two 64 KiB stages


def test_reader_rows_keep_one_permutation_per_thread():
    # a reading thread (512 per workgroup, 32 chunks per row) steps rows by 16:
    # the permutation of its chunk is the same for all the rows it copies
    for r0 in range(16):
        assert len({swz(r0 + i * 16) for i in range(16)}) == 1

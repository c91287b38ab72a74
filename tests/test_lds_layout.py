"""CPU model of the d = 128 forward kernel's LDS tile layout (lin_offset in
fa_device.h): a tile of R rows is R/4 pieces of 1 KiB, piece p holding rows
p, p + R/4, p + 2R/4, p + 3R/4 as whole 256-byte rows, pieces PS bytes apart
(1040 for K and the query tile, 1088 for V).

Checks the properties the kernel relies on: the map is a bijection into the
tile's bytes; one asynchronous copy (64 lanes x 16 bytes to consecutive LDS
addresses) fills one piece and reads whole rows from HBM; the MFMA row read
and the transposed read are a per-lane base plus a lane-independent offset
(the immediates the kernel uses); both reads are free of LDS bank conflicts
(16 lanes of 16 bytes, 32 lanes of 8 bytes, over 64 banks of 4 bytes); and
the transposed read hands each lane the elements the 32x32x16 MFMA A operand
expects.
"""

PK, PV = 1040, 1088


def off(row, chunk, rows, ps):
    return (row % (rows // 4)) * ps + 256 * (row // (rows // 4)) + 16 * chunk


def test_bijective_and_in_bounds():
    for rows, ps in ((64, PK), (64, PV), (128, PK)):
        seen = {off(r, c, rows, ps) for r in range(rows) for c in range(16)}
        assert len(seen) == rows * 16
        assert min(seen) == 0 and max(seen) + 16 <= rows // 4 * ps
    # the query tile fits one K + V buffer
    assert 128 // 4 * PK <= 64 // 4 * PK + 64 // 4 * PV


def test_copy_piece_is_one_dma_and_whole_rows():
    for rows, ps in ((64, PK), (64, PV), (128, PK)):
        for p in range(rows // 4):
            for lane in range(64):
                row, chunk = p + (rows // 4) * (lane >> 4), lane & 15
                assert off(row, chunk, rows, ps) == p * ps + 16 * lane
            # each 16-lane group reads one row's 256 contiguous bytes, in order
            for g in range(4):
                src = [(p + (rows // 4) * (lane >> 4), lane & 15) for lane in range(16 * g, 16 * g + 16)]
                assert len({r for r, _ in src}) == 1
                assert [c for _, c in src] == list(range(16))


def test_row_read_base_plus_immediate_and_conflict_free():
    for rows in (64, 128):
        base = [off(l & 31, l >> 5, rows, PK) for l in range(64)]
        for r0 in range(0, rows, 32):
            for kk in range(8):
                ad = [off(r0 + (l & 31), 2 * kk + (l >> 5), rows, PK) for l in range(64)]
                imm = 256 * (r0 // (rows // 4)) + 32 * kk
                assert all(a == b + imm for a, b in zip(ad, base))
                for ph in range(4):
                    groups = [(a % 256) // 16 for a in ad[16 * ph: 16 * ph + 16]]
                    assert len(set(groups)) == 16


def _tr(r0, c0, lane, hi):
    gi, hg, g16 = lane & 15, (lane >> 5) & 1, (lane >> 4) & 1
    row = r0 + 4 * hg + (gi >> 2) + (8 if hi else 0)
    col = c0 + 16 * g16 + 4 * (gi & 3)
    return row, col, off(row, col // 8, 64, PV) + (col & 4) * 2


def test_transposed_read_base_plus_immediate_conflict_free_and_operand_layout():
    base = [_tr(0, 0, l, False)[2] for l in range(64)]
    for kc in range(4):
        for db in range(4):
            for hi in (False, True):
                ad = [_tr(16 * kc, 32 * db, l, hi)[2] for l in range(64)]
                imm = 256 * kc + 64 * db + (8 * PV if hi else 0)
                assert all(a == b + imm for a, b in zip(ad, base))
                for half in range(2):
                    granules = [(a % 256) // 8 for a in ad[32 * half: 32 * half + 32]]
                    assert len(set(granules)) == 32
                # ds_read_b64_tr_b16: in each 16-lane group, lane i gets element
                # i%4 of the 8 bytes lane 4e + i/4 read; the operand wants column
                # c0 + l%32 at row r0 + 4*(l/32) + e (+8 for the second read)
                for l in range(64):
                    for e in range(4):
                        src = (l & ~15) + 4 * e + (l & 15) // 4
                        row, col, _ = _tr(16 * kc, 32 * db, src, hi)
                        assert col + (l & 15) % 4 == 32 * db + (l & 31)
                        assert row == 16 * kc + 4 * (l >> 5) + e + (8 if hi else 0)

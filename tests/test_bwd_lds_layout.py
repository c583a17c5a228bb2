"""CPU model of the backward kernels' LDS layout (host-side index math).

The backward kernels keep streamed tiles (Q and dO for dK/dV; K and V for
dQ) in natural row order in LDS, with the 16-byte chunks of row r
XOR-swizzled by f(r), a rotation of the row's low bits:
    16+ chunks per row (d = 128):  f(r) = ((r & 3) << 2) | ((r >> 2) & 3)
     8 chunks per row (d = 64):    f(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
Two kinds of reads use the same tile:
  * row fragments (ds_read_b128): lane L reads row 32 blk + L % 32, logical
    chunk 2 s + L // 32 (an MFMA A operand with the contraction over d);
  * transposed fragments (two ds_read_b64_tr_b16): the contraction runs
    over tile rows in the order of a 32x32 MFMA accumulator, lane half h
    and step t holding rows 16 t + 8 w + 4 h + (0..3), w = 0, 1.
The model checks that every lane gets the (row, column) elements the MFMA
needs and that both reads are free of bank conflicts (64 banks x 4 bytes;
b128 in passes of 16 lanes, 8-byte reads in passes of 32 lanes).
"""
import collections

import pytest


def f_rot(D, r):
    if D // 8 >= 16:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


def tile_cells(D, rows):
    cpr = D // 8
    cells = {}
    for p in range(rows * cpr):
        row = p // cpr
        lc = (p % cpr) ^ f_rot(D, row)
        for e in range(8):
            cells[p * 8 + e] = (row, lc * 8 + e)
    return cells


def row_frag_addr(D, blk, s, lane):
    """Kernel: rfo[s] + blk * 32 * D."""
    col, h = lane % 32, lane // 32
    return blk * 32 * D + col * D + (((2 * s + h) ^ f_rot(D, col)) * 8)


def tr_frag_addrs(D, blk, t, db, w):
    """Kernel: (32 blk + 16 t + 8 w) * D + tlane[w][db & 3]."""
    out = []
    for lane in range(64):
        g16, rr = lane >> 4, lane & 15
        vh, vdh, vi, vq = g16 >> 1, g16 & 1, rr >> 2, rr & 3
        lrow = 4 * vh + vi                       # row within the 8-row group
        lc = 4 * db + 2 * vdh + (vq >> 1)
        # f of row 32 blk + 16 t + 8 w + lrow depends on (8 w + lrow) & 15 only
        pc = lc ^ f_rot(D, 8 * w + lrow)
        out.append((32 * blk + 16 * t + 8 * w) * D + (lrow) * D + pc * 8 + (vq & 1) * 4)
    return out


def tr16(addresses, cells):
    rows = [[cells[a + c] for c in range(4)] for a in addresses]
    return [[rows[16 * (l // 16) + (l % 16) // 4 + 4 * i][l % 4] for i in range(4)]
            for l in range(64)]


def bank_cycles(elem_addrs, nbytes, pass_lanes):
    tot = 0
    for p in range(0, 64, pass_lanes):
        banks = collections.defaultdict(set)
        for a in elem_addrs[p:p + pass_lanes]:
            for w in range(nbytes // 4):
                word = a // 2 + w
                banks[word % 64].add(word)
        tot += max(len(s) for s in banks.values())
    return tot


@pytest.mark.parametrize("D,rows", [(64, 64), (128, 64), (128, 32)])
def test_row_fragments(D, rows):
    cells = tile_cells(D, rows)
    for blk in range(rows // 32):
        for s in range(D // 16):
            addrs = [row_frag_addr(D, blk, s, lane) for lane in range(64)]
            for lane in range(64):
                got = [cells[addrs[lane] + e] for e in range(8)]
                want = [(32 * blk + lane % 32, 16 * s + 8 * (lane // 32) + e) for e in range(8)]
                assert got == want
            assert bank_cycles(addrs, 16, 16) == 4


@pytest.mark.parametrize("D,rows", [(64, 64), (128, 64), (128, 32)])
def test_transposed_fragments(D, rows):
    cells = tile_cells(D, rows)
    for blk in range(rows // 32):
        for t in range(2):
            for db in range(D // 32):
                halves = []
                for w in range(2):
                    a = tr_frag_addrs(D, blk, t, db, w)
                    assert bank_cycles(a, 8, 32) == 2
                    halves.append(tr16(a, cells))
                for lane in range(64):
                    h = lane // 32
                    got = halves[0][lane] + halves[1][lane]
                    # accumulator element i = 8 t + e of lane half h is row
                    # 8 (i // 4) + 4 h + i % 4 of the 32-row block
                    want = [(32 * blk + 8 * ((8 * t + e) // 4) + 4 * h + (8 * t + e) % 4,
                             32 * db + lane % 32) for e in range(8)]
                    assert got == want, (D, blk, t, db, lane)

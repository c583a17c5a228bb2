"""CPU model of the FP8 forward kernel's LDS tiles (fa_fp8_kernel.hip).

Restates the kernel's address formulas and checks, with no GPU:
  * the tile copies (16 bytes per lane into a swizzled layout) write every
    (row, 16-byte chunk) of a 128 x 128-byte tile exactly once;
  * each K fragment holds, in lane (key, h), the d-bytes 64 s + 32 h + b of
    its key row, the order in which the wave keeps Q;
  * the four 8-bit transposed reads of a V^T fragment give lane (d, h) the
    32 keys of a 64-key chunk in the order in which the P operand packs the
    S^T accumulator (byte b: 32-key block b / 16, element b % 16, element e
    of lane half h being key 8 (e / 4) + 4 h + e % 4);
  * both read kinds are free of LDS bank conflicts (64 banks of 4 bytes;
    16-byte reads are served 16 lanes at a time, 8-byte reads 32 at a time).

The 8-bit transposed read's lane mapping is the one measured on gfx950: in
each 16-lane group, lane j receives byte j % 8 of the 8-byte pieces
addressed by lanes 2 i + j // 8, for i = 0..7 in order.
"""
import itertools

D = 128            # bytes per row (d = 128, one byte per element)
BN = 128           # keys per tile
NW = 8             # waves per workgroup
NS, NMB, NPC, NDB = D // 64, BN // 32, BN // 64, D // 32


def fk(r):
    return (r >> 1) & 7


def fv(r):
    return (((r >> 1) & 1) | (((r >> 3) & 1) << 1)) << 1


def logical(addr, f):
    """Physical tile byte address -> (row, logical byte column)."""
    row, rest = divmod(addr, D)
    pch, t = divmod(rest, 16)
    return row, (pch ^ f(row)) * 16 + t


def test_copies_cover_each_tile_once():
    for f in (fk, fv):
        seen = set()
        for w, i, lane in itertools.product(range(NW), range(BN * D // 1024 // NW), range(64)):
            pbyte = (w + NW * i) * 1024 + 16 * lane
            row, pch = divmod(pbyte, D)
            pch //= 16
            lc = pch ^ f(row)                 # the logical chunk this lane copies
            assert 0 <= lc < D // 16
            # it lands where the layout puts logical chunk lc of that row
            assert row * D + (lc ^ f(row)) * 16 == pbyte
            seen.add((row, lc))
        assert len(seen) == BN * D // 16


def k_frag_addrs(mb, s, lane):
    col, h = lane & 31, lane >> 5
    return [mb * 32 * D + col * D + ((4 * s + 2 * h + t) ^ fk(col)) * 16 for t in (0, 1)]


def test_k_fragment_contents():
    for mb, s, lane in itertools.product(range(NMB), range(NS), range(64)):
        col, h = lane & 31, lane >> 5
        got = []
        for a in k_frag_addrs(mb, s, lane):
            row, c0 = logical(a, fk)
            got += [(row, c0 + t) for t in range(16)]
        want = [(32 * mb + col, 64 * s + 32 * h + b) for b in range(32)]
        assert got == want


def test_k_reads_conflict_free():
    for mb, s, t in itertools.product(range(NMB), range(NS), (0, 1)):
        for p in range(4):                      # 16 lanes per pass
            groups = {(k_frag_addrs(mb, s, lane)[t] // 16) % 16 for lane in range(16 * p, 16 * p + 16)}
            assert len(groups) == 16


def v_lane_addr(pc, db, u, lane):
    g, s16 = lane >> 4, lane & 15
    va, ve, vhh, vg1, vt = s16 >> 3, (s16 >> 1) & 3, g >> 1, g & 1, s16 & 1
    vrow = 8 * va + 4 * vhh + ve
    vfh = fv(vrow) >> 1
    vlane = vrow * D + 32 * (db ^ vfh) + 16 * vg1 + 8 * vt
    return (64 * pc + 32 * (u >> 1) + 16 * (u & 1)) * D + vlane


def p_operand_key(pc, h, b):
    """Key (within the tile) of byte b of lane half h of P's operand."""
    mb, e = 2 * pc + b // 16, b % 16
    return 32 * mb + 8 * (e // 4) + 4 * h + e % 4


def test_v_fragment_matches_p_operand():
    for pc, db in itertools.product(range(NPC), range(NDB)):
        recv = {}
        for u in range(4):
            pieces = {L: logical(v_lane_addr(pc, db, u, L), fv) for L in range(64)}
            for L in range(64):
                row, c0 = pieces[L]
                assert c0 % 8 == 0
            for L in range(64):
                g, j = L >> 4, L & 15
                for i in range(8):
                    src = 16 * g + 2 * i + j // 8
                    row, c0 = pieces[src]
                    recv[(L, 8 * u + i)] = (row, c0 + j % 8)
        for L in range(64):
            h = L >> 5
            for b in range(32):
                assert recv[(L, b)] == (p_operand_key(pc, h, b), 32 * db + L % 32)


def test_v_reads_conflict_free():
    for pc, db, u in itertools.product(range(NPC), range(NDB), range(4)):
        for p in range(2):                      # 32 lanes per pass
            banks = []
            for L in range(32 * p, 32 * p + 32):
                a = v_lane_addr(pc, db, u, L)
                banks += [(a // 4) % 64, (a // 4 + 1) % 64]
            assert len(set(banks)) == 64


def test_reads_stay_in_tile():
    for mb, s, lane in itertools.product(range(NMB), range(NS), range(64)):
        assert all(0 <= a and a + 16 <= BN * D for a in k_frag_addrs(mb, s, lane))
    for pc, db, u, lane in itertools.product(range(NPC), range(NDB), range(4), range(64)):
        a = v_lane_addr(pc, db, u, lane)
        assert 0 <= a and a + 8 <= BN * D

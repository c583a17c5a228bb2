"""CPU model of the direct-load kernel's LDS layout (host-side index math).

The bf16 kernel copies K and V tiles into LDS with global_load_lds (lane L
of a wave instruction lands at 16-byte chunk L of a 1 KB block), XOR-swizzles
the 16-byte chunks of every row, and reads the V^T operand with
ds_read_b64_tr_b16, whose lane semantics (checked on the GPU with an
in-bounds probe) are: in each 16-lane group, lane l receives element l % 4 of
the 8-byte rows supplied by lanes (l % 16) // 4 + 4 i, i = 0..3.

This test re-derives, for every lane, which (key, d) elements the K and V^T
MFMA operands end up holding, and checks them against the operand layout the
kernel assumes (v_mfma_f32_32x32x16_bf16: lane L holds row L % 32 and eight
contraction elements for lane half L // 32; the P^T operand of lane half h,
element e, of key block mb and step t is key mb*32 + 16h + 8t + e).  The
formulas mirror the kernel's; a mismatch here means an addressing bug.
"""
import pytest


def k_slot_key(r):
    """Key stored in LDS slot r of a 32-row block."""
    return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3)


def swz_mask(D):
    cpr = D // 8
    return min(cpr, 16) - 1


def lds_tile(D, BN, tensor):
    """Physical element offset -> (key, d) after the DMA copies."""
    cpr = D // 8
    swz = swz_mask(D)
    nblk = BN * cpr // 64
    cells = {}
    for blk in range(nblk):
        for lane in range(64):
            p = blk * 64 + lane
            row = p // cpr
            lc = (p % cpr) ^ (row & swz)
            if tensor == "K":
                key = (row & ~31) | k_slot_key(row & 31)
            else:
                key = row
            for e in range(8):
                cells[p * 8 + e] = (key, lc * 8 + e)
    assert len(cells) == BN * D
    return cells


@pytest.mark.parametrize("D,BN", [(64, 128), (128, 128), (128, 64), (256, 64), (256, 32)])
def test_k_operand_layout(D, BN):
    cells = lds_tile(D, BN, "K")
    swz = swz_mask(D)
    for mb in range(BN // 32):
        for st in range(D // 16):
            for lane in range(64):
                col, half = lane % 32, lane // 32
                kfo = col * D + (((2 * st + half) ^ (col & swz)) * 8)
                a = mb * 32 * D + kfo
                got = [cells[a + e] for e in range(8)]
                # S^T accumulator row r = col of key block mb holds key
                # mb*32 + k_slot_key(col); contraction d = 16 st + 8 half + e
                want = [(mb * 32 + k_slot_key(col), 16 * st + 8 * half + e)
                        for e in range(8)]
                assert got == want, (D, BN, mb, st, lane)


def tr16(addresses, cells):
    """ds_read_b64_tr_b16 over 64 lanes; addresses are element offsets."""
    rows = [[cells[a + c] for c in range(4)] for a in addresses]
    out = []
    for l in range(64):
        g = l // 16
        out.append([rows[16 * g + (l % 16) // 4 + 4 * i][l % 4] for i in range(4)])
    return out


@pytest.mark.parametrize("D,BN", [(64, 128), (128, 128), (128, 64), (256, 64), (256, 32)])
def test_vt_operand_layout(D, BN):
    cells = lds_tile(D, BN, "V")
    swz = swz_mask(D)
    for mb in range(BN // 32):
        for t in range(2):
            for db in range(D // 32):
                halves = []
                for w in range(2):
                    addrs = []
                    for lane in range(64):
                        g16, rr = lane >> 4, lane & 15
                        vh, vdh, vi, vq = g16 >> 1, g16 & 1, rr >> 2, rr & 3
                        vlane = ((16 * vh + vi) * D
                                 + (((2 * vdh + (vq >> 1)) ^ vi) & 3) * 8
                                 + (vq & 1) * 4)
                        tw = ((8 * t + 4 * w) & swz) >> 2
                        cofs = (mb * 32 + 8 * t + 4 * w) * D + ((db ^ tw) << 2) * 8
                        addrs.append(cofs + vlane)
                    halves.append(tr16(addrs, cells))
                for lane in range(64):
                    got = halves[0][lane] + halves[1][lane]
                    h = lane // 32
                    want = [(mb * 32 + 16 * h + 8 * t + e, db * 32 + lane % 32)
                            for e in range(8)]
                    assert got == want, (D, BN, mb, t, db, lane, got[:3], want[:3])


def test_old_mask_would_fail_for_d256():
    """The unbounded swizzle mask (row & (D/8 - 1)) mixes the lane half into
    the compile-time offset at d = 256; the model must detect that."""
    D, BN = 256, 64
    cpr = D // 8
    cells = {}
    for blk in range(BN * cpr // 64):
        for lane in range(64):
            p = blk * 64 + lane
            row = p // cpr
            lc = (p % cpr) ^ (row & (cpr - 1))
            for e in range(8):
                cells[p * 8 + e] = (row, lc * 8 + e)
    bad = 0
    for lane in range(64):
        g16, rr = lane >> 4, lane & 15
        vh, vdh, vi, vq = g16 >> 1, g16 & 1, rr >> 2, rr & 3
        vlane = ((16 * vh + vi) * D + (((2 * vdh + (vq >> 1)) ^ vi) & 3) * 8
                 + (vq & 1) * 4)
        tw = ((8 * 0 + 4 * 0) & (cpr - 1)) >> 2
        a = 0 * D + ((0 ^ tw) << 2) * 8 + vlane
        if any(cells[a + c][1] // 32 != 0 for c in range(4)):
            bad += 1
    assert bad > 0

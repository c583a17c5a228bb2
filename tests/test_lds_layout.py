"""CPU model of the direct-load kernel's LDS layout (host-side index math).

The bf16 kernel copies K and V tiles into LDS with global_load_lds (lane L
of a wave instruction lands at 16-byte chunk L of a 1 KB block), swizzles
the 16-byte chunks of every row (logical chunk lc of row r sits at physical
chunk lc ^ f(r), with one f for K and another for V), and reads the V^T
operand with ds_read_b64_tr_b16, whose lane semantics (checked on the GPU
with an in-bounds probe) are: in each 16-lane group, lane l receives element
l % 4 of the 8-byte rows supplied by lanes (l % 16) // 4 + 4 i, i = 0..3.

These tests re-derive, for every lane, which (key, d) elements the K and V^T
MFMA operands end up holding, and check them against the operand layout the
kernel assumes (v_mfma_f32_32x32x16_bf16: lane L holds row L % 32 and eight
contraction elements for lane half L // 32; the P^T operand of lane half h,
element e, of key block mb and step t is key mb*32 + 16h + 8t + e).  They
also count LDS bank cycles per read under a model of the LDS (64 banks of
4 bytes; ds_read_b128 served 16 lanes per pass, 8-byte reads 32 lanes per
pass; a pass costs the largest number of distinct words in one bank), which
matched the bank-conflict counter of the previous layout.  The formulas
mirror the kernel's; a mismatch here means an addressing bug.
"""
import collections

import pytest

SHAPES = [(64, 128), (64, 64), (128, 128), (128, 64), (256, 64), (256, 32)]


def k_slot_key(r):
    """Key stored in LDS slot r of a 32-row block."""
    return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3)


def f_k(D, r):
    return (r & 15) if D // 8 >= 16 else ((r >> 1) & 7)


def f_v(D, r):
    return ((r & 3) << 2) if D // 8 >= 16 else (((r >> 1) & 1) << 2)


def lds_tile(D, BN, tensor, f):
    """Physical element offset -> (key, d) after the copies."""
    cpr = D // 8
    cells = {}
    for p in range(BN * cpr):   # block p // 64, lane p % 64
        row = p // cpr
        lc = (p % cpr) ^ f(D, row)
        key = (row & ~31) | k_slot_key(row & 31) if tensor == "K" else row
        for e in range(8):
            cells[p * 8 + e] = (key, lc * 8 + e)
    assert len(cells) == BN * D
    return cells


def k_addresses(D, mb, st, f=f_k):
    """Element offsets of the K fragment reads (kernel: kfo[st] + mb*32*D)."""
    out = []
    for lane in range(64):
        col, half = lane % 32, lane // 32
        out.append(mb * 32 * D + col * D + (((2 * st + half) ^ f(D, col)) * 8))
    return out


def v_addresses(D, mb, t, db, w, f=f_v):
    """Element offsets of one ds_read_b64_tr_b16 (kernel: cofs + vlane[db & 3])."""
    nvl = min(D // 32, 4)
    out = []
    for lane in range(64):
        g16, rr = lane >> 4, lane & 15
        vh, vdh, vi, vq = g16 >> 1, g16 & 1, rr >> 2, rr & 3
        x = db & (nvl - 1)
        lc = 4 * x + 2 * vdh + (vq >> 1)
        vlane = (16 * vh + vi) * D + (lc ^ f(D, vi)) * 8 + (vq & 1) * 4
        cofs = (mb * 32 + 8 * t + 4 * w) * D + (db & ~3) * 32
        out.append(cofs + vlane)
    return out


@pytest.mark.parametrize("D,BN", SHAPES)
def test_k_operand_layout(D, BN):
    cells = lds_tile(D, BN, "K", f_k)
    for mb in range(BN // 32):
        for st in range(D // 16):
            addrs = k_addresses(D, mb, st)
            for lane in range(64):
                col, half = lane % 32, lane // 32
                got = [cells[addrs[lane] + e] for e in range(8)]
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


@pytest.mark.parametrize("D,BN", SHAPES)
def test_vt_operand_layout(D, BN):
    cells = lds_tile(D, BN, "V", f_v)
    for mb in range(BN // 32):
        for t in range(2):
            for db in range(D // 32):
                halves = [tr16(v_addresses(D, mb, t, db, w), cells) for w in range(2)]
                for lane in range(64):
                    got = halves[0][lane] + halves[1][lane]
                    h = lane // 32
                    want = [(mb * 32 + 16 * h + 8 * t + e, db * 32 + lane % 32)
                            for e in range(8)]
                    assert got == want, (D, BN, mb, t, db, lane, got[:3], want[:3])


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


@pytest.mark.parametrize("D,BN", SHAPES)
def test_reads_are_bank_conflict_free(D, BN):
    for mb in range(BN // 32):
        for st in range(D // 16):
            assert bank_cycles(k_addresses(D, mb, st), 16, 16) == 4
        for t in range(2):
            for db in range(D // 32):
                for w in range(2):
                    assert bank_cycles(v_addresses(D, mb, t, db, w), 8, 32) == 2


def test_model_detects_conflicts_of_a_single_swizzle():
    """The earlier layout (one XOR swizzle r & 15 for both tensors) puts the
    4 rows of a transposed read on the same 16 banks; the model must see the
    resulting 4-way conflict."""
    same = lambda D, r: r & 15
    assert bank_cycles(v_addresses(128, 0, 0, 0, 0, f=same), 8, 32) == 8
    assert bank_cycles(k_addresses(64, 0, 0, f=lambda D, r: r & 7), 16, 16) == 8


@pytest.mark.parametrize("D", [64, 128, 256])
def test_k_fragment_offsets_repeat_every_8_steps(D):
    """The kernel keeps one K-fragment lane offset per d step only for the
    first 8 steps: the swizzle touches the low 4 bits of the chunk index
    2s + half, so step s + 8 reads 16 chunks (128 elements) further."""
    ns = D // 16
    for lane in range(64):
        col, half = lane & 31, lane >> 5
        for st in range(ns):
            want = col * D + ((2 * st + half) ^ f_k(D, col)) * 8
            got = col * D + ((2 * (st % 8) + half) ^ f_k(D, col)) * 8 + (st // 8) * 128
            assert got == want, (D, lane, st)

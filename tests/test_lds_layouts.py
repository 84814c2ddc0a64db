"""The LDS layouts of the HIP kernels, checked exhaustively on the CPU.

Every kernel that stages tiles in LDS with direct global -> LDS loads stores
rows unpadded and permutes the 16-byte chunks of each row with an XOR, so
that its read patterns meet distinct banks.  This file restates each
permutation and each read pattern (lane -> byte address, written from the
kernels' documented layouts) and checks, for every row, lane and offset the
kernels use:
* the permutation is a bijection of the chunk slots of a row;
* a tile written the way the direct loads write it (byte t of the tile
  holds, from row t / RB, the chunk that slot (t % RB) / 16 is assigned)
  reads back, through every read pattern, exactly the element that pattern
  asks for -- including the offsets the kernels fold into immediates;
* the read patterns meet no bank twice within one phase.

Bank model (CDNA LDS, 64 banks of 4 bytes, so one 256-byte bank line): a
wave's LDS access is served in phases of 256 bytes, i.e. 16 lanes of a
16-byte read, 32 lanes of an 8-byte (transposing) read, 64 lanes of a
4-byte read; a phase is conflict-free when no bank is touched twice.
No GPU is involved: these are facts about integer maps.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest

BANKS = 64
LINE = 256


def bank_degree(addrs, width):
    """Largest number of accesses one bank receives within one phase, for
    lane byte addresses `addrs` (in lane order) each reading `width` bytes."""
    per_phase = LINE // width
    worst = 0
    for p0 in range(0, len(addrs), per_phase):
        count = {}
        for a in addrs[p0:p0 + per_phase]:
            for w in range(0, width, 4):
                bank = ((a + w) // 4) % BANKS
                count[bank] = count.get(bank, 0) + 1
        worst = max(worst, max(count.values()))
    return worst


def write_tile(rows, rb, swz):
    """LDS image of a tile of `rows` rows of `rb` bytes written by the direct
    loads: the 16-byte slot s of row r holds the row's chunk s ^ swz(r).
    Returns an int array [rows * rb] whose byte at address a holds the tile
    byte index (row * rb + byte within the row) stored there."""
    lds = np.full(rows * rb, -1, np.int64)
    for t in range(0, rows * rb, 16):
        r, s = t // rb, (t % rb) // 16
        c = s ^ swz(r)
        assert 0 <= c < rb // 16, "permutation leaves the row"
        lds[t:t + 16] = r * rb + c * 16 + np.arange(16)
    assert (lds >= 0).all()
    assert np.array_equal(np.sort(lds), np.arange(rows * rb)), "tile bytes lost or duplicated"
    return lds


def check_bijection(rb, swz, rows):
    n = rb // 16
    for r in range(rows):
        assert sorted(c ^ swz(r) for c in range(n)) == list(range(n)), (rb, r)


# ---------------------------------------------------------------------------
# attention forward (direct-to-LDS stages of K and V; page "Multi-head
# attention and self-attention", Definition: S = c Q K^T, Z = A V)
# ---------------------------------------------------------------------------

def k_swizzle(rb):
    """Chunk c of a K row r sits in slot c ^ ((r / (256 / RB)) mod (RB / 16))."""
    rpb = 1 if rb >= 256 else 256 // rb
    return lambda r: (r // rpb) % (rb // 16)


def v_swizzle(rb):
    """Chunk c of a V row r sits in slot c ^ 4 ((r / (256 / RB)) mod (RB / 64))
    for rows of 128 or 256 bytes; other widths are unpermuted."""
    if rb in (128, 256):
        rpb = 256 // rb
        return lambda r: 4 * ((r // rpb) % (rb // 64))
    return lambda r: 0


FWD_K_RB = [64, 128, 256]          # d_h = 32, 64, 128 (two-byte elements)
FWD_V_RB = [64, 128, 192, 256]     # d_vh = 32, 64, 96, 128
BN = 64                            # keys per block


@pytest.mark.parametrize("rb", FWD_K_RB)
def test_forward_k_rows(rb):
    """Score operand: lane (l32 = lane % 32, g = lane / 32) reads 16 bytes of
    K row 32 kb + l32 at chunk 2 c + g; the kernel computes the address from
    l32 only and adds 32 kb rows as an immediate."""
    swz = k_swizzle(rb)
    check_bijection(rb, swz, BN)
    lds = write_tile(BN, rb, swz)
    kch = rb // 32                  # k-chunk pairs of the score product
    for kb in range(BN // 32):
        for c in range(kch):
            addrs = []
            for lane in range(64):
                l32, g = lane % 32, lane // 32
                base = l32 * rb + ((2 * c + g) ^ swz(l32)) * 16
                a = base + 32 * kb * rb
                row, chunk = 32 * kb + l32, 2 * c + g
                assert np.array_equal(lds[a:a + 16], row * rb + chunk * 16 + np.arange(16))
                addrs.append(a)
            assert bank_degree(addrs, 16) == 1, (rb, kb, c)


def v_read_addrs(rb, swz, d, off_rows):
    """Transposing read of V^T: lane reads 8 bytes of row off_rows + 4 g +
    (lane % 16) / 4 at column 32 d + 16 ((lane / 16) % 2) + 4 (lane % 4); the
    kernel's base depends on the row through 4 g + (lane % 16) / 4 only."""
    out = []
    for lane in range(64):
        g = lane // 32
        vr = 4 * g + (lane % 16) // 4
        scol = 16 * ((lane // 16) % 2) + 4 * (lane % 4)
        col = 32 * d + scol
        base = vr * rb + ((col // 8) ^ swz(vr)) * 16 + (col % 8) * 2
        out.append((base + off_rows * rb, off_rows + vr, col))
    return out


@pytest.mark.parametrize("rb", FWD_V_RB)
def test_forward_v_rows(rb):
    swz = v_swizzle(rb)
    check_bijection(rb, swz, BN)
    lds = write_tile(BN, rb, swz)
    for kb, st, h in itertools.product(range(BN // 32), range(2), range(2)):
        for d in range(rb // 64):
            reads = v_read_addrs(rb, swz, d, 32 * kb + 16 * st + 8 * h)
            for a, row, col in reads:
                assert np.array_equal(lds[a:a + 8], row * rb + col * 2 + np.arange(8))
            assert bank_degree([a for a, _, _ in reads], 8) == 1, (rb, kb, st, h, d)


@pytest.mark.parametrize("rb", FWD_K_RB)
def test_forward_k_swizzle_needed(rb):
    """Without the permutation the K reads of 16 rows at one chunk would pile
    up on the same banks (the permutation is doing work)."""
    addrs = [(lane % 32) * rb + (lane // 32) * 16 for lane in range(64)]
    assert bank_degree(addrs, 16) > 1


def test_forward_mask_tile():
    """Boolean mask tile: 128 query rows x 64 key bytes per stage.  Window w
    (1 KB) holds rows 16 w .. 16 w + 15; lane i fills row 16 w + i / 4, slot
    i % 4, from the row's chunk (i % 4) ^ ((row / 4) mod 4).  The mask step's
    lane (l32, g) of wave wv reads 4 bytes of row 32 wv + l32 at chunk
    2 kb + a / 2 (slot chunk ^ ((row / 4) mod 4)), byte 8 (a mod 2) + 4 g:
    keys 32 kb + 8 a + 4 g .. + 3."""
    rows, rb = 128, 64
    swz = lambda r: (r // 4) % 4
    check_bijection(rb, swz, rows)
    # the windows' lanes, as the kernel forms them
    lds = np.full(rows * rb, -1, np.int64)
    for w in range(rows * rb // 1024):
        for i in range(64):
            t = w * 1024 + 16 * i
            row, slot = t // 64, (t % 64) // 16
            assert row == 16 * w + i // 4 and slot == i % 4
            chunk = slot ^ ((row >> 2) & 3)
            lds[t:t + 16] = row * rb + chunk * 16 + np.arange(16)
    assert np.array_equal(np.sort(lds), np.arange(rows * rb))
    for wv in range(4):
        for kb, a in itertools.product(range(2), range(4)):
            addrs = []
            for lane in range(64):
                l32, g = lane % 32, lane // 32
                mr = 32 * wv + l32
                c = 2 * kb + a // 2
                addr = mr * 64 + (c ^ ((mr >> 2) & 3)) * 16 + 8 * (a & 1) + 4 * g
                key = 32 * kb + 8 * a + 4 * g
                assert np.array_equal(lds[addr:addr + 4], mr * rb + key + np.arange(4))
                addrs.append(addr)
            # 32 rows at one chunk: each bank at most twice (unpermuted: 8 times)
            assert bank_degree(addrs, 4) == 2
            flat = [(32 * wv + lane % 32) * 64 + (2 * kb + a // 2) * 16 + 8 * (a & 1)
                    + 4 * (lane // 32) for lane in range(64)]
            assert bank_degree(flat, 4) == 8


def test_forward_mask_window_reads_and_tests():
    """The mask step reads dwords (kb, a) in pairs: chunk c = 2 kb + h at base
    row * 64 + 16 (c ^ ((row / 4) mod 4)) + 4 g, dword a = 2 h + e at + 8 e
    (one two-dword LDS read per chunk), the addresses of the per-dword form
    above.  Its window tests: no allowed entry iff the OR of the dwords is 0;
    every entry allowed (skip the per-score test) only if bit 0 is set in
    every byte of the AND: exact for 0 / 1 bytes, and for other bytes never
    true unless every byte is nonzero (so a false answer only costs the
    per-score test)."""
    for wv, lane, kb, h, e in itertools.product(range(4), range(64), range(2), range(2),
                                                range(2)):
        l32, g = lane % 32, lane // 32
        mr = 32 * wv + l32
        c, a = 2 * kb + h, 2 * h + e
        base = mr * 64 + (c ^ ((mr >> 2) & 3)) * 16 + 4 * g
        direct = mr * 64 + ((2 * kb + a // 2) ^ ((mr >> 2) & 3)) * 16 + 8 * (a & 1) + 4 * g
        assert base + 8 * e == direct
    rng = np.random.default_rng(7)

    def tests(words):
        all_and = np.bitwise_and.reduce(words)
        any_set = np.bitwise_or.reduce(words)
        return any_set == 0, (all_and & 0x01010101) == 0x01010101

    def as_words(b):
        return b.reshape(-1, 4).astype(np.uint32) @ np.array([1, 1 << 8, 1 << 16, 1 << 24],
                                                               dtype=np.uint32)
    for trial in range(4000):
        kind = trial % 4
        if kind == 0:
            b = (rng.random(32) < 0.97).astype(np.uint8)              # 0 / 1
        elif kind == 1:
            b = np.ones(32, np.uint8)
        elif kind == 2:
            b = np.zeros(32, np.uint8)
            b[rng.integers(32)] = rng.integers(0, 2) * rng.integers(1, 256)
        else:
            b = rng.integers(0, 256, 32).astype(np.uint8) * (rng.random(32) < 0.95)
        none_allowed, full = tests(as_words(b))
        assert none_allowed == (not b.any())
        if full:
            assert b.all()
        if kind <= 1:
            assert full == bool(b.all())


def bias_fast_offsets(q0, wave, n_k, k0):
    """Byte offsets of the bias-tile direct loads on the fast path (every
    row of the tile below n_q, every key of the block below n_k): window q
    of lane i is 4 (row0 + 4 q) n_k + 4 k0 + 16 (c0 ^ 4 (q mod 4)),
    row0 = q0 + 32 wave + i / 16, c0 = (i mod 16) ^ (i / 16)."""
    out = {}
    for q in range(8):
        for lane in range(64):
            row0 = q0 + 32 * wave + lane // 16
            c0 = (lane % 16) ^ (lane // 16)
            out[q, lane] = 4 * (row0 + 4 * q) * n_k + 4 * k0 + 16 * (c0 ^ (4 * (q % 4)))
    return out


@pytest.mark.parametrize("n_k,k0,q0", [(64, 0, 0), (4096, 1984, 3968), (192, 64, 128)])
def test_forward_bias_tile(n_k, k0, q0):
    """Additive bias tile: 128 query rows x 64 fp32 keys (256 bytes a row)
    per block, each wave its own 32 rows in eight 1 KB windows.  Window q of
    wave w holds rows 32 w + 4 q + i / 16; lane i fills slot i mod 16 of its
    row from the row's chunk (i mod 16) ^ (row mod 16) (four keys).  The
    mask step's lane (l32, g) reads row 32 w + l32, chunk 8 kb + 2 a + g at
    slot chunk ^ (l32 mod 16): keys 32 kb + 8 a + 4 g .. + 3."""
    rows, rb = 128, 256
    swz = lambda r: r % 16
    check_bijection(rb, swz, rows)
    for wave in range(4):
        fast = bias_fast_offsets(q0, wave, n_k, k0)
        # the tile as the windows write it: byte t of window q of this wave
        # holds global byte fast[q, t / 16] + t mod 16 of the bias matrix
        lds = np.full(32 * rb, -1, np.int64)
        for q in range(8):
            for lane in range(64):
                row = 32 * wave + 4 * q + lane // 16
                chunk = (lane % 16) ^ (row % 16)
                # the direct (clamped-path) form of the same offset
                direct = 4 * ((q0 + row) * n_k + k0 + 4 * chunk)
                assert fast[q, lane] == direct
                t = q * 1024 + 16 * lane
                assert t // rb == row - 32 * wave and (t % rb) // 16 == lane % 16
                lds[t:t + 16] = direct + np.arange(16)
        assert (lds >= 0).all()
        want_rows = 4 * (q0 + 32 * wave + np.arange(32))[:, None] * n_k + 4 * k0
        want = (want_rows + np.arange(rb)[None, :]).ravel()
        assert np.array_equal(np.sort(lds), np.sort(want)), "tile bytes lost or duplicated"
        for kb, a in itertools.product(range(2), range(4)):
            addrs = []
            for lane in range(64):
                l32, g = lane % 32, lane // 32
                c = 8 * kb + 2 * a + g
                addr = l32 * rb + (c ^ (l32 % 16)) * 16
                key = 32 * kb + 8 * a + 4 * g
                row = q0 + 32 * wave + l32
                assert np.array_equal(lds[addr:addr + 16],
                                      4 * (row * n_k + k0 + key) + np.arange(16))
                addrs.append(addr)
            # 16 rows at one chunk per phase: distinct 16-byte bank groups
            # (unpermuted, all 16 lanes would meet one group)
            assert bank_degree(addrs, 16) == 1
            flat = [(lane % 32) * rb + (8 * kb + 2 * a + lane // 32) * 16 for lane in range(64)]
            assert bank_degree(flat, 16) == 16


# ---------------------------------------------------------------------------
# attention backward (direct-load stages read both row-wise and transposed)
# ---------------------------------------------------------------------------

def bwd_swizzle(rb):
    """Chunk c of row r sits in slot c ^ (4 (h mod q) + (h / q) mod 4), h the
    row's 256-byte bank line and q the 64-byte quarters per row."""
    rpb, q, ck = 256 // rb, rb // 64, rb // 16
    return lambda r: ((r // rpb) % q * 4 + (r // rpb // q) % 4) % ck


@pytest.mark.parametrize("rb", [128, 256])
def test_backward_tiles(rb):
    """Row reads: lane (l32, g) reads 16 bytes of row 32 sb + l32 at chunk
    2 c + g.  Transposing reads: rows 32 sb + 16 st + 8 hh + 4 g +
    (lane % 16) / 4, columns 32 d + scol; the kernel's bases depend on the row
    through 8 hh + 4 g + (lane % 16) / 4 (hh has its own base)."""
    swz = bwd_swizzle(rb)
    rows = 64
    check_bijection(rb, swz, rows)
    lds = write_tile(rows, rb, swz)
    for sb in range(rows // 32):
        for c in range(rb // 32):
            addrs = []
            for lane in range(64):
                l32, g = lane % 32, lane // 32
                a = l32 * rb + ((2 * c + g) ^ swz(l32)) * 16 + 32 * sb * rb
                assert np.array_equal(lds[a:a + 16],
                                      (32 * sb + l32) * rb + (2 * c + g) * 16 + np.arange(16))
                addrs.append(a)
            assert bank_degree(addrs, 16) == 1, (rb, sb, c)
    for sb, st, hh in itertools.product(range(rows // 32), range(2), range(2)):
        for d in range(rb // 64):
            addrs = []
            for lane in range(64):
                g = lane // 32
                vr = 8 * hh + 4 * g + (lane % 16) // 4
                col = 32 * d + 16 * ((lane // 16) % 2) + 4 * (lane % 4)
                a = vr * rb + ((col // 8) ^ swz(vr)) * 16 + (col % 8) * 2 + (32 * sb + 16 * st) * rb
                row = 32 * sb + 16 * st + vr
                assert np.array_equal(lds[a:a + 8], row * rb + col * 2 + np.arange(8))
                addrs.append(a)
            assert bank_degree(addrs, 8) == 1, (rb, sb, st, hh, d)


# ---------------------------------------------------------------------------
# projection GEMMs (X tile read row-wise, W tile read transposed)
# ---------------------------------------------------------------------------

GEMM_LAYOUTS = {
    # name: (A row bytes, A permutation, W row bytes, W permutation)
    "dma": (64, lambda r: (r >> 2) & 3, 256, lambda r: 4 * (r & 3)),
    "dma_wide": (128, lambda r: (r >> 1) & 7, 512, lambda r: 4 * (r & 3)),
}


@pytest.mark.parametrize("name", sorted(GEMM_LAYOUTS))
def test_gemm_a_tile(name):
    """A rows (k contiguous): the load of window q of wave wv fills rows
    16 (or 8) per instruction; lane (l32, g) reads 16 bytes of row
    wm 128 + 32 i + l32 at chunk 2 kc + g (32 i an immediate)."""
    rb, swz, _, _ = GEMM_LAYOUTS[name]
    rows = 256
    check_bijection(rb, swz, rows)
    lds = write_tile(rows, rb, swz)
    # the per-lane write form the kernels use
    per_instr = 1024 // rb
    for t in range(0, rows * rb, 16):
        instr, lane = t // 1024, (t % 1024) // 16
        assert t // rb == instr * per_instr + lane // (rb // 16)
        assert (t % rb) // 16 == lane % (rb // 16)
    for wm, i in itertools.product(range(2), range(4)):
        for kc in range(rb // 32):
            addrs = []
            for lane in range(64):
                l32, g = lane % 32, lane // 32
                r = wm * 128 + l32
                a = r * rb + ((2 * kc + g) ^ swz(r)) * 16 + 32 * i * rb
                row = wm * 128 + 32 * i + l32
                assert np.array_equal(lds[a:a + 16], row * rb + (2 * kc + g) * 16 + np.arange(16))
                addrs.append(a)
            assert bank_degree(addrs, 16) == 1, (name, wm, i, kc)


@pytest.mark.parametrize("name", sorted(GEMM_LAYOUTS))
def test_gemm_w_tile(name):
    """W rows (n contiguous, one k per row): lane reads 8 bytes of k row
    16 kc + 8 g + (lane % 16) / 4 + 4 h at columns wn 64 + 32 j +
    16 ((lane / 16) mod 2) + 4 (lane mod 4); kc and h are immediates."""
    _, _, rb, swz = GEMM_LAYOUTS[name]
    rows = 32
    check_bijection(rb, swz, rows)
    lds = write_tile(rows, rb, swz)
    ncols = rb // 2
    for kc, h in itertools.product(range(rows // 16), range(2)):
        for wn, j in itertools.product(range(ncols // 64), range(2)):
            addrs = []
            for lane in range(64):
                g = lane // 32
                kr = 8 * g + (lane % 16) // 4
                col = wn * 64 + 32 * j + 16 * ((lane // 16) % 2) + 4 * (lane % 4)
                a = kr * rb + ((col >> 3) ^ swz(kr)) * 16 + (col & 7) * 2 + (16 * kc + 4 * h) * rb
                row = 16 * kc + 4 * h + kr
                assert np.array_equal(lds[a:a + 8], row * rb + col * 2 + np.arange(8))
                addrs.append(a)
            assert bank_degree(addrs, 8) == 1, (name, kc, h, wn, j)

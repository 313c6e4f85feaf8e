"""Host check of the DMA kernels' LDS slot swizzles for B in the [K, N]
layout (the rule the kernel source states beside `bswz` in gemm_dma.hip):

* each B row's swizzle is a bijection of its 16-byte slots;
* it uses only bits of the row index k that the transposing reads' immediate
  row offsets never change (16-bit inputs: offsets 4 r and 32 ks; fp8 8 r), so
  a lane may compute the slot once for row k;
* the 16 lanes of each quarter-wave of a transposing read touch 32 distinct
  4-byte banks (of 64), for every column block and row offset; the 32-column
  tile's swizzle keeps each half-wave's 32 lanes on 64 distinct banks too.

The swizzles are restated here from that source, per row width."""
import pytest


def bswz(eb: int, bslots: int, k: int) -> int:
    if eb == 2:
        if bslots >= 16:
            return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1)
        if bslots == 8:
            return ((k & 3) << 1) ^ ((k >> 3) & 1)
        return ((k >> 3) & 1) << 1
    if bslots >= 16:
        return (k & 7) << 1
    if bslots == 8:
        return k & 7
    return (k & 3) ^ ((k >> 2) & 1)


# (element bytes, tile columns): the [K, N] B rows of the DMA tiles
CASES = [(2, 256), (2, 64), (2, 32), (1, 256)]


@pytest.mark.parametrize("eb,tbn", CASES)
def test_swizzle_is_a_bijection_per_row(eb, tbn):
    bslots = tbn * eb // 16
    for k in range(128 // eb):
        assert sorted(c ^ bswz(eb, bslots, k) for c in range(bslots)) == list(range(bslots))


@pytest.mark.parametrize("eb,tbn", CASES)
def test_swizzle_ignores_the_read_offsets(eb, tbn):
    # a lane's first row: k = 8 grp + t (t < 4) for 16-bit inputs, 32 grp + t
    # (t < 8) for fp8; the reads add the offsets below
    bslots = tbn * eb // 16
    if eb == 2:
        # the narrow tiles' 256-byte stages have four k-steps
        bases = [8 * g + t for g in range(4) for t in range(4)]
        offsets = [4 * r + 32 * ks for r in range(2) for ks in range(4 if tbn <= 64 else 2)]
    else:
        bases = [32 * g + t for g in range(4) for t in range(8)]
        offsets = [8 * r for r in range(4)]
    for k in bases:
        for off in offsets:
            assert bswz(eb, bslots, k + off) == bswz(eb, bslots, k), (k, off)


def _read_addrs(eb, tbn, j, off):
    """Byte addresses (8 bytes each) of the 64 lanes of one transposing read of
    column block j at row offset off (the 16x16 steps: 16-bit 4 K rows per
    lane group, fp8 8 K rows)."""
    brow = tbn * eb
    bslots = brow // 16
    out = []
    for lane in range(64):
        grp, gi = lane >> 4, lane & 15
        if eb == 2:
            t, q = gi >> 2, gi & 3
            n, k = j * 16 + 4 * q, 8 * grp + t
            a = k * brow + (((n >> 3) ^ bswz(eb, bslots, k)) << 4) + (q & 1) * 8
        else:
            t, q = gi >> 1, gi & 1
            n, k = j * 16 + 8 * q, 32 * grp + t
            a = k * brow + (((n >> 4) ^ bswz(eb, bslots, k)) << 4) + q * 8
        out.append(a + off * brow)
    return out


def _distinct_banks(addrs, lanes):
    for h in range(64 // lanes):
        banks = [(a // 4 + d) % 64 for a in addrs[lanes * h:lanes * (h + 1)] for d in range(2)]
        if len(set(banks)) != 2 * lanes:
            return False
    return True


@pytest.mark.parametrize("eb,tbn", CASES)
def test_transposing_reads_hit_distinct_banks(eb, tbn):
    kbytes = 256 if tbn <= 64 else 128  # K bytes per stage
    offsets = [4 * r + 32 * ks for r in range(2) for ks in range(kbytes // 64)] if eb == 2 else \
        [8 * r for r in range(4)]
    for j in range(tbn // 16):
        for off in offsets:
            addrs = _read_addrs(eb, tbn, j, off)
            assert max(addrs) + 8 <= (kbytes // eb) * tbn * eb  # inside the stage's B block
            assert _distinct_banks(addrs, 16), (j, off)
            if tbn == 32:
                assert _distinct_banks(addrs, 32), (j, off)


def test_the_32_column_swizzle_separates_rows_k_and_k_plus_8():
    """Unswizzled 64-byte rows put rows k and k + 8 of a half-wave on the same
    banks; the swizzle's slot swap separates them."""
    def addrs(swz):
        out = []
        for lane in range(64):
            grp, gi = lane >> 4, lane & 15
            t, q = gi >> 2, gi & 3
            n, k = 4 * q, 8 * grp + t
            out.append(k * 64 + (((n >> 3) ^ (bswz(2, 4, k) if swz else 0)) << 4) + (q & 1) * 8)
        return out
    assert not _distinct_banks(addrs(False), 32)
    assert _distinct_banks(addrs(True), 32)


def aswz(row_bytes: int, r: int) -> int:
    return r & 15 if row_bytes == 256 else (r >> 1) & 7


@pytest.mark.parametrize("row_bytes", [128, 256])
def test_a_rows_quarter_waves_hit_distinct_banks(row_bytes):
    """A (and B given transposed): the 16 lanes of a quarter-wave read 16
    bytes of rows base + 0 .. 15 at one slot c; the row swizzle puts them on
    64 distinct banks, for every slot c and block row base."""
    slots = row_bytes // 16
    for base in range(0, 64, 16):
        for c in range(slots):
            assert sorted(c2 ^ aswz(row_bytes, base) for c2 in range(slots)) == list(range(slots))
            banks = []
            for lb in range(16):
                r = base + lb
                a = r * row_bytes + ((c ^ aswz(row_bytes, lb)) << 4)
                banks += [(a // 4 + d) % 64 for d in range(4)]
            assert len(set(banks)) == 64, (row_bytes, base, c)

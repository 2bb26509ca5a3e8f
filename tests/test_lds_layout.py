"""Model of the LDS tile layouts the 16-bit kernels address (runs without a GPU).

The kernels' own addressing is exercised for real by the GPU parity tests;
this file checks the layout design those kernels follow, in a bank model of
the gfx950 LDS: 64 banks of 4 bytes; a 16-byte row read (ds_read_b128) is
served 16 lanes per cycle, a transposing 8-byte read (ds_read_b64_tr_b16)
32 lanes per cycle.  The model agrees with the hardware counters: the
forward's tiles and the swizzled backward tiles count 0 bank conflicts, the
backward's former 304-byte padded rows counted one conflict cycle per LDS
instruction.

Checked: (1) the direct-to-LDS loads place every (row, 16-byte chunk) of a
tile exactly once, (2) the row reads and transposing reads find the chunks
the unswizzled addressing would, (3) neither read pattern has a bank
conflict, for every padded head_dim of the 16-bit kernels.
"""
import pytest


def tr_row_stride(min_bytes):
    st = (min_bytes + 15) // 16 * 16
    while st % 256 not in (64, 192):
        st += 16
    return st


def swz_chunk(p, row):
    return (p & ~3) | ((p & 3) ^ ((row >> 2) & 3))


def conflict_free(addrs, nbytes):
    banks = [((a + i) // 4) % 64 for a in addrs for i in range(0, nbytes, 4)]
    return len(set(banks)) == len(banks)


def row_read_addrs(R, st, block):
    """16-byte reads of k-step st: lane (l32, hi) reads row block*32 + l32, chunk 2 st + hi."""
    out = []
    for lane in range(64):
        l32, hi = lane & 31, lane >> 5
        sw = (l32 >> 2) & 3
        base = l32 * R + 16 * ((hi ^ sw ^ 2) if st & 1 else (hi ^ sw))
        out.append(base + block * 32 * R + 64 * (st >> 1))
    return out


def tr_read_addrs(R, u, db, upper):
    """Transposing reads: rows 16 u + 4 hi + s16 / 4 (+ 8), chunk 4 db + 2 ((lane / 16) % 2) + (s16 % 4) / 2."""
    out = []
    for lane in range(64):
        hi, s16 = lane >> 5, lane & 15
        t_row = 4 * hi + (s16 >> 2)
        t_ch = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1)
        half = 8 * (s16 & 1)
        if upper:
            base = (t_row + 8) * R + 16 * (t_ch ^ hi ^ 2) + half
        else:
            base = t_row * R + 16 * (t_ch ^ hi) + half
        out.append(base + 16 * u * R + 64 * db)
    return out


@pytest.mark.parametrize("d", [32, 64, 80, 96, 128, 256])
@pytest.mark.parametrize("rows", [32, 64])
def test_swizzled_dual_read_tile(d, rows):
    dblk = (d + 31) // 32
    ksteps = d // 16
    R = tr_row_stride(dblk * 64)
    slots = R // 16
    # (1) the loads fill slot p of row r with chunk swz_chunk(p, r): a bijection per row
    for r in range(rows):
        chunks = [swz_chunk(p, r) for p in range(4 * dblk)]
        assert sorted(chunks) == list(range(4 * dblk))

    def chunk_at(addr):
        r, off = divmod(addr, R)
        p, b = divmod(off, 16)
        assert p < slots
        return r, swz_chunk(p, r), b

    # (2) + (3) row reads
    for block in range(rows // 32):
        for st in range(ksteps):
            addrs = row_read_addrs(R, st, block)
            for lane, a in enumerate(addrs):
                r, ch, b = chunk_at(a)
                assert (r, ch, b) == (block * 32 + (lane & 31), 2 * st + (lane >> 5), 0)
            for g in range(4):
                assert conflict_free(addrs[16 * g:16 * g + 16], 16)
    # transposing reads
    for u in range(rows // 16):
        for db in range(dblk):
            for upper in (False, True):
                addrs = tr_read_addrs(R, u, db, upper)
                for lane, a in enumerate(addrs):
                    hi, s16 = lane >> 5, lane & 15
                    row = 16 * u + 4 * hi + (s16 >> 2) + (8 if upper else 0)
                    byte = (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2 + 64 * db
                    assert chunk_at(a) == (row, byte // 16, byte % 16)
                for g in range(2):
                    assert conflict_free(addrs[32 * g:32 * g + 32], 8)


def test_padded_stride_without_swizzle_conflicts_on_transposing_reads():
    """The former 304-byte rows (row reads conflict-free) put the rows of a
    transposing read into overlapping bank windows: the swizzle is needed."""
    R = 304
    addrs = []
    for lane in range(32):
        s16 = lane & 15
        addrs.append((s16 >> 2) * R + (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2)
    assert not conflict_free(addrs, 8)
    rows16 = [r * R for r in range(16)]
    assert conflict_free(rows16, 16)


@pytest.mark.parametrize("d", [32, 64, 80, 96, 128])
def test_forward_tile_strides(d):
    """Forward: K rows 2d + 16 bytes (row reads only), V rows 64/192 mod 256 (transposing only)."""
    kr = 2 * d + 16
    dblk = (d + 31) // 32
    vr = tr_row_stride(dblk * 64)
    for c in range(d // 8):
        assert conflict_free([r * kr + 16 * c for r in range(16)], 16)
    for db in range(dblk):
        addrs = []
        for lane in range(32):
            s16 = lane & 15
            addrs.append((s16 >> 2) * vr + (16 * ((lane >> 4) & 1) + 4 * (s16 & 3)) * 2 + 64 * db)
        assert conflict_free(addrs, 8)


def lds_swizzle(r, rowb):
    """Slot permutation of the chunks of an unpadded row of `rowb` bytes (the
    head_dim-64/128 forward with K/V loads two tiles ahead): chunk c of row r
    sits at slot c ^ lds_swizzle(r, rowb)."""
    if rowb == 256:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_swizzled_unpadded_rows(d):
    """head_dim 64 / 128, 64-row K and V tiles at 2 d bytes per row without
    padding: (1) the direct-to-LDS loads of 1 KiB place every chunk exactly
    once; (2) the K row reads and the V transposing reads, addressed as the
    kernel does, find the chunks of the unswizzled layout; (3) neither
    conflicts."""
    R, rows, ksteps, dblk = 2 * d, 64, d // 16, d // 32
    nch = R // 16
    # (1) load slot -> (row, chunk): slot p of row r holds chunk p ^ lds_swizzle(r)
    placed = set()
    for inst in range(rows * nch // 64):
        for lane in range(64):
            slot = inst * 64 + lane
            r, p = divmod(slot, nch)
            placed.add((r, p ^ lds_swizzle(r, R)))
    assert placed == {(r, c) for r in range(rows) for c in range(nch)}

    def chunk_at(addr):
        r, off = divmod(addr, R)
        p, b = divmod(off, 16)
        return r, p ^ lds_swizzle(r, R), b

    # (2) + (3) K row reads: lane (l32, hi), k-step st, 32-row block kb2
    for kb2 in range(2):
        for st in range(ksteps):
            addrs = []
            for lane in range(64):
                l32, hi = lane & 31, lane >> 5
                a = l32 * R + 16 * ((2 * st + hi) ^ lds_swizzle(l32, R)) + kb2 * 32 * R
                assert chunk_at(a) == (kb2 * 32 + l32, 2 * st + hi, 0)
                addrs.append(a)
            for g in range(4):
                assert conflict_free(addrs[16 * g:16 * g + 16], 16)
    # V transposing reads: 16-row group u, 32-dim block db, rows r and r + 8
    for u in range(rows // 16):
        for db in range(dblk):
            for upper in (False, True):
                addrs = []
                for lane in range(64):
                    hi, s16 = lane >> 5, lane & 15
                    r = 4 * hi + (s16 >> 2) + (8 if upper else 0)
                    byte = 32 * ((lane >> 4) & 1) + 8 * (s16 & 3)
                    c = (byte >> 4) + 4 * db
                    a = r * R + 16 * (c ^ lds_swizzle(r, R)) + (byte & 15) + 16 * u * R
                    assert chunk_at(a) == (16 * u + r, c, byte & 15)
                    addrs.append(a)
                for g in range(2):
                    assert conflict_free(addrs[32 * g:32 * g + 32], 8)

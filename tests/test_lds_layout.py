"""Host-side checks of the LDS tile layouts the kernels use.

The kernels read 16-bit K/V/Q/dO tiles from LDS in two patterns: 16-byte row
fragments (16 lanes, 16 consecutive tile rows, one 16-byte chunk each) and
transpose reads (ds_read_b64_tr_b16: half a wave reads 8 bytes per lane from
4 consecutive tile rows x 4 aligned 16-byte chunks, two 8-byte halves each).
The layout maps (the XOR swizzle of unpadded rows, lds_swizzle in
csrc/fa_device.h, and the row permutation of padded rows, lds_row) are
stated below as the kernels define them; the tests check the properties the
kernels rely on, under a model of 64 LDS banks of 4 bytes:

* every map is a bijection of a tile's 16-byte chunks;
* both read patterns touch distinct banks (no bank conflicts);
* the transpose-read address splits into a lane part (computed once per
  kernel) plus base * D for every tile row base that is a multiple of 16,
  which is how the d = 128 forward and dQ kernels form those addresses.
"""
import itertools

import pytest

BANKS = 64  # 4-byte banks


def lds_swizzle(d, r):
    # physical 16-byte chunk = logical chunk ^ lds_swizzle(r)
    if d == 64:  # 128-byte rows: two rows per bank sweep
        return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
    return ((r & 3) << 2) | ((r >> 2) & 3)  # 256-byte rows


def lds_row(r):
    # padded tiles: tile row r sits at LDS row lds_row(r) (bits 0-1 and 2-3 swapped)
    return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3)


def swz_elem(d, row, col):
    """Element offset of (row, col) in an unpadded swizzled tile (8 elements per chunk)."""
    return row * d + (((col >> 3) ^ lds_swizzle(d, row)) << 3) + (col & 7)


def tr_lane_addrs(d, base, col0, lane):
    """Element offsets of a lane's two transpose reads (rows base + ..., + 8)."""
    j = lane & 15
    row = base + 4 * (lane >> 5) + (j >> 2)
    col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3)
    return swz_elem(d, row, col), swz_elem(d, row + 8, col)


def banks_of(byte_addr, nbytes):
    return {(byte_addr // 4 + k) % BANKS for k in range(nbytes // 4)}


@pytest.mark.parametrize("d", [64, 128])
def test_swizzle_is_a_bijection_of_chunks(d):
    chunks = d // 8
    for r in range(64):
        phys = {c ^ lds_swizzle(d, r) for c in range(chunks)}
        assert phys == set(range(chunks)), r


@pytest.mark.parametrize("d", [64, 128])
def test_swizzled_row_fragment_reads_are_conflict_free(d):
    # 16 lanes read logical chunk c of 16 consecutive rows (a 16-aligned group)
    for r0 in range(0, 64, 16):
        for c in range(d // 8):
            seen = set()
            for r in range(r0, r0 + 16):
                b = banks_of(2 * swz_elem(d, r, 8 * c), 16)
                assert not (b & seen), (d, r0, c, r)
                seen |= b


def test_swizzled_transpose_reads_are_conflict_free():
    # the transpose reads run on the d = 128 swizzled tiles (direct-to-LDS loads)
    d = 128
    for base in range(0, 64, 16):
        for col0 in range(0, d, 32):
            for which in (0, 1):
                for half in (0, 1):
                    seen = set()
                    for lane in range(32 * half, 32 * half + 32):
                        b = banks_of(2 * tr_lane_addrs(d, base, col0, lane)[which], 8)
                        assert not (b & seen), (base, col0, which, lane)
                        seen |= b
                    assert len(seen) == BANKS


@pytest.mark.parametrize("d", [64, 128])
def test_transpose_address_splits_into_lane_part_and_row_offset(d):
    for lane, col0 in itertools.product(range(64), range(0, d, 32)):
        lane0 = tr_lane_addrs(d, 0, col0, lane)
        for base in range(0, 128, 16):
            got = tr_lane_addrs(d, base, col0, lane)
            assert got == (lane0[0] + base * d, lane0[1] + base * d), (lane, col0, base)


def test_row_permutation_is_a_bijection_within_16_rows():
    for r0 in range(0, 64, 16):
        assert sorted(lds_row(r) for r in range(r0, r0 + 16)) == list(range(r0, r0 + 16))


@pytest.mark.parametrize("d,stride_bytes", [(64, 144), (128, 304)])
def test_padded_permuted_row_fragment_reads_are_conflict_free(d, stride_bytes):
    for r0 in range(0, 64, 16):
        for c in range(d // 8):
            seen = set()
            for r in range(r0, r0 + 16):
                b = banks_of(lds_row(r) * stride_bytes + 16 * c, 16)
                assert not (b & seen), (d, r0, c, r)
                seen |= b


def _padded_transpose_banks(d, stride_bytes, row_map, base, col0, k, hi):
    """Banks of each lane of half a wave for one transpose read of a padded tile: the
    fragment's tile rows base + 4*hi + j/4 (+ 8 for its second read, k = 1), stored
    at LDS row row_map(tile row)."""
    stride = stride_bytes // 2
    out = []
    for lane in range(32 * hi, 32 * hi + 32):
        j = lane & 15
        lrow = row_map(base + 4 * (lane >> 5) + (j >> 2) + 8 * k)
        col = col0 + 16 * ((lane >> 4) & 1) + 4 * (j & 3)
        out.append((lane, lrow, banks_of(2 * (lrow * stride + col), 8)))
    return out


@pytest.mark.parametrize("d,stride_bytes", [(64, 144), (128, 304)])
def test_padded_permuted_transpose_reads_are_conflict_free(d, stride_bytes):
    for base, col0, k, hi in itertools.product(range(0, 64, 16), range(0, d, 32), (0, 1), (0, 1)):
        seen = set()
        for lane, lrow, b in _padded_transpose_banks(d, stride_bytes, lds_row, base, col0, k, hi):
            # the LDS row load_frag_tr_rp addresses for this lane
            assert lrow == base + 4 * ((lane & 15) >> 2) + (lane >> 5) + 2 * k, (lane, k)
            assert not (b & seen), (d, base, col0, k, lane)
            seen |= b


@pytest.mark.parametrize("d,stride_bytes", [(64, 144), (128, 304)])
def test_unpermuted_padded_transpose_reads_conflict(d, stride_bytes):
    # why the permutation exists: rows in tile order at these strides overlap
    conflicts = 0
    for base, col0 in itertools.product(range(0, 64, 16), range(0, d, 32)):
        seen = set()
        for _, _, b in _padded_transpose_banks(d, stride_bytes, lambda r: r, base, col0, 0, 0):
            conflicts += len(b & seen)
            seen |= b
    assert conflicts > 0

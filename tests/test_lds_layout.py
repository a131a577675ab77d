"""Host-side checks of the swizzled LDS tile layout the HIP kernels use.

The swizzle (fa_device.hpp, swz<D> and tile_off<D>) stores the 16-byte chunk
k of tile row r at chunk position k ^ swz(r).  These tests restate that map
and check the properties the kernels rely on:

* it is a permutation of each row's chunks, and the direct HBM->LDS copy
  pattern (tile_offsets) writes every chunk of a tile exactly once;
* the MFMA operand reads (ds_read_b128: 16 lanes read one logical chunk of 16
  consecutive rows) touch 64 distinct 4-byte banks;
* the transposing reads (ds_read_b64_tr_b16: 32 lanes read 4 consecutive
  rows x 32 consecutive columns) touch 64 distinct banks.

LDS is modelled as 64 banks of 4 bytes; a 16-byte read covers 4 banks and an
8-byte read 2.
"""
import itertools

import pytest

BANKS = 64


def swz(D, row):
    if D == 128:
        return ((row & 3) << 2) | ((row >> 2) & 3)
    u = (row >> 1) & 7
    return ((u & 1) << 2) | (u >> 1)


def tile_off(D, row, col):
    """Element offset of (row, col) in a swizzled tile of D-element rows."""
    return row * D + ((((col >> 3) ^ swz(D, row))) << 3) + (col & 7)


def banks(byte_addr, nbytes):
    return {(byte_addr // 4 + i) % BANKS for i in range(nbytes // 4)}


@pytest.mark.parametrize("D", [64, 128])
def test_swizzle_permutes_each_row(D):
    cpr = D // 8
    for row in range(64):
        assert 0 <= swz(D, row) < cpr
        assert sorted(k ^ swz(D, row) for k in range(cpr)) == list(range(cpr))


@pytest.mark.parametrize("D,rows,nt", [(64, 64, 256), (128, 64, 256), (128, 32, 256), (64, 32, 256),
                                       (128, 128, 256), (64, 128, 256)])
def test_copy_pattern_writes_every_chunk_once(D, rows, nt):
    """tile_offsets/load_tile_async: lane `lane` of wave `wave`, copy r, writes the
    physical chunk c = r*NT + wave*64 + lane and reads logical chunk
    (c % CPR) ^ swz(row) of row c / CPR."""
    cpr = D // 8
    per_lane = rows * cpr // nt
    seen = set()
    for r, wave, lane in itertools.product(range(per_lane), range(nt // 64), range(64)):
        c = r * nt + wave * 64 + lane
        row, k = c // cpr, (c % cpr) ^ swz(D, c // cpr)
        # the element the chunk holds lands where tile_off says it should
        assert tile_off(D, row, k * 8) == c * 8
        seen.add((row, k))
    assert len(seen) == rows * cpr


@pytest.mark.parametrize("D", [64, 128])
def test_copy_offsets_repeat_every_copy(D):
    """The copies of one lane step by whole swizzle periods, so their source
    offsets are copy 0's plus a uniform step (load_tile_async relies on it)."""
    cpr, nt = D // 8, 256
    assert (nt // cpr) % 16 == 0
    for wave, lane in itertools.product(range(4), range(64)):
        c0 = wave * 64 + lane
        for r in range(4):
            c = r * nt + c0
            off = (c // cpr) * D + (((c % cpr) ^ swz(D, c // cpr)) << 3)
            off0 = (c0 // cpr) * D + (((c0 % cpr) ^ swz(D, c0 // cpr)) << 3)
            assert off == off0 + r * (nt // cpr) * D


@pytest.mark.parametrize("D", [64, 128])
def test_operand_reads_are_conflict_free(D):
    """ds_read_b128 of an MFMA operand: lane (l32, hi) reads row base + l32,
    logical chunk 2*kk + hi; each group of 16 lanes is one LDS cycle."""
    for base, kk in itertools.product(range(0, 64, 32), range(D // 16)):
        for group in range(4):
            seen = set()
            for lane in range(group * 16, group * 16 + 16):
                l32, hi = lane & 31, lane >> 5
                b = banks(2 * tile_off(D, base + l32, kk * 16 + hi * 8), 16)
                assert not (seen & b), (D, base, kk, group)
                seen |= b
            assert len(seen) == BANKS


@pytest.mark.parametrize("D", [64, 128])
def test_transposing_reads_are_conflict_free(D):
    """ds_read_b64_tr_b16 of V^T / Q^T / dO^T / K^T: lane (j16, dsub, hi)
    points at row base + 8r + 4 hi + j16/4, column dt*32 + 16 dsub +
    4 (j16 % 4); each group of 32 lanes is one LDS cycle."""
    for base, r, dt in itertools.product(range(0, 64, 16), range(2), range(D // 32)):
        for half in range(2):
            seen = set()
            for lane in range(half * 32, half * 32 + 32):
                j16, dsub, hi = lane & 15, (lane >> 4) & 1, lane >> 5
                row = base + 8 * r + 4 * hi + (j16 >> 2)
                col = dt * 32 + 16 * dsub + 4 * (j16 & 3)
                b = banks(2 * tile_off(D, row, col), 8)
                assert not (seen & b), (D, base, r, dt, half)
                seen |= b
            assert len(seen) == BANKS


@pytest.mark.parametrize("D", [64, 128])
def test_operand_read_steps_are_xor(D):
    """The kernels address the operand read of step kk as offset(0) ^ (kk << 5)
    bytes, with offset(0) that of row r, chunk hi (r any tile row, hi 0/1)."""
    for row, hi in itertools.product(range(128), range(2)):
        base = 2 * tile_off(D, row, hi * 8)
        for kk in range(D // 16):
            assert 2 * tile_off(D, row, kk * 16 + hi * 8) == base ^ (kk << 5), (D, row, hi, kk)


@pytest.mark.parametrize("D", [64, 128])
def test_transposing_read_steps_are_xor(D):
    """The kernels address the transposing read of column tile dt as
    offset(0) ^ (dt << 6) bytes, offset(0) that of column 16 dsub + 4 c."""
    for row, dsub, c in itertools.product(range(128), range(2), range(4)):
        col0 = 16 * dsub + 4 * c
        base = 2 * tile_off(D, row, col0)
        for dt in range(D // 32):
            assert 2 * tile_off(D, row, dt * 32 + col0) == base ^ (dt << 6), (D, row, dsub, c, dt)

"""CPU model of the shared-prefix tile's LDS layout (csrc/pa_shared.hip:
sh_swizzle, sh_off, the direct loads' lane placement and the operand
reads).  Every direct load fills 8 rows x 128 bytes (whole lines of global
memory), lane l landing at byte 16 l; the MFMA operand reads of K and q
(ds_read_b128, 16 lanes per LDS pass) and the transposing V reads
(ds_read_b64_tr_b16, 32 lanes per pass) must find exactly the bytes they
want and, within one pass, touch distinct banks (64 banks of 4 bytes)."""

import pytest

KT = 32     # keys (rows) per tile
PART = KT * 128


def swizzle(row):
    x = (row >> 1) & 7
    return ((x & 1) << 2) | (x & 2) | (x >> 2)


def off(row, b):
    return (b >> 7) * PART + row * 128 + ((((b >> 4) & 7) ^ swizzle(row)) << 4) + (b & 15)


def placement(D):
    """LDS byte -> (row, byte of the row) after the tile's direct loads."""
    lds = {}
    for p in range(2 * D // 128):
        for i in range(4):
            for lane in range(64):
                row = i * 8 + (lane >> 3)
                src = p * 128 + (((lane & 7) ^ swizzle(row)) << 4)
                for k in range(16):
                    lds[p * PART + i * 1024 + 16 * lane + k] = (row, src + k)
    return lds


def k_read(lane, ks):
    li, h = lane & 31, lane >> 5
    return (ks >> 2) * PART + off(li, (2 * (ks & 3) + h) * 16), (li, (2 * ks + h) * 16)


def v_read(lane, s2, dt, hi):
    g16, k4, q4 = lane >> 4, (lane >> 2) & 3, lane & 3
    vrow, vch = 4 * (g16 >> 1) + k4, (g16 & 1) * 2 + (q4 >> 1)
    addr = s2 * 16 * 128 + (dt >> 1) * PART + off(vrow + 8 * hi, (dt & 1) * 64 + vch * 16 + (q4 & 1) * 8)
    return addr, (s2 * 16 + vrow + 8 * hi, dt * 64 + vch * 16 + (q4 & 1) * 8)


@pytest.mark.parametrize("D", [64, 128])
def test_loads_fill_the_tile_once(D):
    assert len(placement(D)) == KT * 2 * D


@pytest.mark.parametrize("D", [64, 128])
def test_operand_reads_find_their_bytes(D):
    lds = placement(D)
    for lane in range(64):
        for ks in range(D // 16):
            a, (row, b) = k_read(lane, ks)
            assert [lds[a + k] for k in range(16)] == [(row, b + k) for k in range(16)]
        for s2 in range(2):
            for dt in range(D // 32):
                for hi in range(2):
                    a, (row, b) = v_read(lane, s2, dt, hi)
                    assert [lds[a + k] for k in range(8)] == [(row, b + k) for k in range(8)]


@pytest.mark.parametrize("D", [64, 128])
def test_operand_reads_are_free_of_bank_conflicts(D):
    for ks in range(D // 16):
        for p in range(4):  # 16 lanes x 16 bytes per pass
            assert len({(k_read(l, ks)[0] % 256) // 16 for l in range(16 * p, 16 * p + 16)}) == 16
    for s2 in range(2):
        for dt in range(D // 32):
            for hi in range(2):
                for p in range(2):  # 32 lanes x 8 bytes per pass
                    assert len({(v_read(l, s2, dt, hi)[0] % 256) // 8 for l in range(32 * p, 32 * p + 32)}) == 32


def test_a_plausible_mistake_is_caught():
    """Without the swizzle, 16 rows' same chunk share one bank group."""
    assert len({((ks_row * 128) % 256) // 16 for ks_row in range(16)}) < 16

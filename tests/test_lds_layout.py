"""CPU emulation of the forward kernel's LDS layouts and operand gathers.

The kernel (csrc/fwd_kernel.hip, csrc/kernel_common.h) stages K and V tiles
in LDS in XOR-swizzled 16-byte units, fills them with direct global-to-LDS
loads, and gathers matrix-instruction operands with plain and transposing
LDS reads.  Each index formula is restated here and its result checked
against what the matrix instruction needs:

  * v_mfma_f32_32x32x16 (16-bit): lane l supplies row l % 32 of A (B: column
    l % 32) and k = 8 (l / 32) + e for its elements e < 8;
  * v_mfma_scale_f32_32x32x64_f8f6f4 (8-bit): lane l supplies k =
    32 (l / 32) + t for its bytes t < 32;
  * ds_read_b64_tr_b16: within a 16-lane group, output lane i element e is
    element i % 4 of the 8 bytes read by source lane 4 e + i / 4;
  * ds_read_b64_tr_b8: within a 16-lane group, output lane i byte j is byte
    i % 8 of the 8 bytes read by source lane 2 j + i / 8 (the mapping the
    kernel's comments record from an on-device probe).

Checked: the swizzles are bijections; the DMA of a tile writes every unit of
the swizzled layout exactly once; the K fragments, the 16-bit V^T fragments
and the e4m3 V^T fragments hold exactly the keys and columns that the S and
P operands they meet expect (P's key order is the order in which the S
accumulator leaves it); and the reads meet the bank-spread properties the
code states.  No GPU is used.
"""
import pytest

BN = 64   # keys per tile


def swz(row, row_bytes):
    if row_bytes == 256:
        return ((row & 3) << 2) | ((row >> 2) & 3)
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3)


def lds_offset(row, unit, row_bytes):
    return row * row_bytes + ((unit ^ swz(row, row_bytes)) << 4)


def v8_swz(row):
    return (row & 3) | (((row >> 3) & 1) << 2)


def bank_group(addr):
    """The 16-byte unit position of an LDS byte address within a 256-byte window."""
    return (addr >> 4) & 15


def conflict_free(addrs, nbytes):
    """LDS model: 64 banks of 4 bytes, 256 bytes served per pass, so a pass
    takes 256 / nbytes lanes of an nbytes-per-lane read; within each pass the
    lanes' bytes must fall in distinct banks."""
    per_pass = 256 // nbytes
    for p0 in range(0, len(addrs), per_pass):
        banks = [((a + b) >> 2) & 63 for a in addrs[p0:p0 + per_pass] for b in range(0, nbytes, 4)]
        if len(set(banks)) != len(banks):
            return False
    return True


@pytest.mark.parametrize("row_bytes", [256, 128])
def test_swizzle_is_a_bijection_per_row_and_spreads_rows(row_bytes):
    units = row_bytes // 16
    for r in range(BN):
        assert sorted(u ^ swz(r, row_bytes) for u in range(units)) == list(range(units))
    # 16 consecutive rows reading the same logical unit hit 16 distinct positions
    # (the K fragment reads: 16 lanes, 16 rows, one unit each)
    for r0 in range(0, BN, 16):
        for u in range(units):
            pos = [lds_offset(r0 + i, u, row_bytes) for i in range(16)]
            if row_bytes == 256:
                assert len({bank_group(a) for a in pos}) == 16
            else:   # two rows per 256-byte window: 16 distinct units over the 8 windows' halves
                assert len({(a >> 4) & 31 for a in pos}) == 16


@pytest.mark.parametrize("row_bytes,waves", [(256, 4), (128, 4)])
def test_dma_writes_the_swizzled_layout(row_bytes, waves):
    # one DMA instruction fills 1 KB: lane L writes LDS bytes 16 L .. 16 L + 15
    # of its block and fetches the global unit that the swizzle puts there
    units = row_bytes // 16
    tile_bytes = BN * row_bytes
    blocks = tile_bytes // 1024
    seen = {}
    for wave in range(waves):
        for i in range(blocks // waves):
            blk = wave * (blocks // waves) + i
            for lane in range(64):
                pos = blk * 64 + lane
                row, phys = pos // units, pos % units
                logical = phys ^ swz(row, row_bytes)        # dma_col: the unit fetched from global
                lds = blk * 1024 + 16 * lane
                assert lds == lds_offset(row, logical, row_bytes)
                assert (row, logical) not in seen
                seen[(row, logical)] = lds
    assert len(seen) == BN * units


def p_keys_16bit(lane, j):
    """Keys (relative to the half) that lane `lane` holds in k-step j of the
    packed 16-bit P, in element order: the S^T accumulator's rows for this
    lane's column are 8 (r / 4) + 4 (l / 32) + r % 4, packed in pairs."""
    h = lane // 32
    keys = [8 * (r // 4) + 4 * h + r % 4 for r in range(16)]     # accumulator element r
    return keys[8 * j:8 * j + 8]


def test_packed_p_matches_the_16bit_mfma_k_layout():
    # a k-step's 16 keys are covered once by the two lane halves together
    for j in range(2):
        k_of = {}
        for lane in range(64):
            for e, key in enumerate(p_keys_16bit(lane, j)):
                k = 8 * (lane // 32) + e
                assert k_of.setdefault((lane % 32, k), key) == key
        for col in range(32):
            assert sorted(k_of[(col, k)] for k in range(16)) == list(range(16 * j, 16 * j + 16))


@pytest.mark.parametrize("d", [64, 128])
def test_v_transposing_reads_16bit(d):
    row_bytes = 2 * d
    # V tile: element (key, col) identified by the pair itself
    lds = {}
    for key in range(BN):
        for col in range(d):
            lds[lds_offset(key, col // 8, row_bytes) + 2 * (col % 8)] = (key, col)
    for c in range(d // 32):
        for hb in range(2):
            for j in range(2):
                base = (32 * hb + 16 * j) * row_bytes
                for r8 in range(2):
                    # per lane: the address of its 8-byte read (va[r8][c])
                    src = []
                    for lane in range(64):
                        g, sl = lane >> 4, lane & 15
                        vrow = 4 * (g >> 1) + (sl >> 2) + 8 * r8
                        dcol = 32 * c + 16 * (g & 1) + 4 * (sl & 3)
                        src.append(base + lds_offset(vrow, dcol >> 3, row_bytes) + (dcol & 7) * 2)
                    assert conflict_free(src, 8)
                    for lane in range(64):
                        g, i = lane >> 4, lane & 15
                        got = []
                        for e in range(4):
                            s = 16 * g + 4 * e + i // 4
                            got.append(lds[src[s] + 2 * (i % 4)])
                        # A operand of O^T += V^T P^T: row d = lane % 32 of column block c,
                        # elements 4 r8 .. 4 r8 + 3 of the lane's k-step keys
                        want_keys = p_keys_16bit(lane, j)[4 * r8:4 * r8 + 4]
                        assert got == [(32 * hb + k, 32 * c + lane % 32) for k in want_keys]


@pytest.mark.parametrize("d", [64, 128])
def test_k_fragment_reads_16bit(d):
    # S^T = K Q^T: lane l reads row l % 32 of the half, unit 2 st + l / 32,
    # i.e. d = 16 st + 8 (l / 32) .. + 7: A's k = 8 (l / 32) + e within k-step st,
    # matching Q^T fragment st of the same lane (d = 16 st + 8 half + e)
    row_bytes = 2 * d
    for hb in range(2):
        for st in range(d // 16):
            addrs = []
            for lane in range(64):
                col, half = lane & 31, lane >> 5
                ka = lds_offset(col, 2 * st + half, row_bytes)
                addr = 32 * hb * row_bytes + ka
                key, unit = divmod(addr, row_bytes)
                unit_logical = (unit // 16) ^ swz(key % BN, row_bytes)
                assert key == 32 * hb + col
                assert unit_logical == 2 * st + half
                addrs.append(addr)
            assert conflict_free(addrs, 16)


def p_keys_e4m3(lane):
    """Keys of the tile that lane `lane` holds in its 32 bytes of e4m3 P:
    half a's 16 accumulator rows, then half b's."""
    h = lane // 32
    return [32 * (t // 16) + 8 * ((t % 16) // 4) + 4 * h + t % 4 for t in range(32)]


def test_e4m3_p_matches_the_8bit_mfma_k_layout():
    k_of = {}
    for lane in range(64):
        for t, key in enumerate(p_keys_e4m3(lane)):
            k_of[(lane % 32, 32 * (lane // 32) + t)] = key
    for col in range(32):
        assert sorted(k_of[(col, k)] for k in range(64)) == list(range(64))


def test_v_transposing_reads_e4m3():
    d, row_bytes = 128, 128
    lds = {}
    for key in range(BN):
        for col in range(d):
            unit, byte = divmod(col, 16)
            lds[key * row_bytes + ((unit ^ v8_swz(key)) << 4) + byte] = (key, col)
    assert len(lds) == BN * d
    # the DMA of an e4m3 V tile (v_off): lane L of block blk fetches the
    # global unit that v8_swz puts at LDS bytes blk * 1024 + 16 L
    seen = set()
    for blk in range(BN * row_bytes // 1024):
        for lane in range(64):
            row, phys = divmod(blk * 64 + lane, row_bytes // 16)
            unit = phys ^ v8_swz(row)
            assert blk * 1024 + 16 * lane == row * row_bytes + ((unit ^ v8_swz(row)) << 4)
            seen.add((row, unit))
    assert len(seen) == BN * row_bytes // 16
    for c in range(d // 32):
        va8 = []
        for lane in range(64):
            g, sl = lane >> 4, lane & 15
            j = sl >> 1
            row = 8 * (j >> 2) + 4 * (g >> 1) + (j & 3)
            unit = 2 * c + (g & 1)
            va8.append(row * row_bytes + ((unit ^ v8_swz(row)) << 4) + 8 * (sl & 1))
        for rr in range(4):
            src = [a + 2048 * rr for a in va8]
            # the 8 rows a 16-lane group reads sit on 8 distinct 16-byte positions,
            # and each 32-lane pass of the 8-byte reads is free of bank conflicts
            for g in range(4):
                assert len({bank_group(src[16 * g + 2 * jj]) for jj in range(8)}) == 8
            assert conflict_free(src, 8)
            for lane in range(64):
                g, i = lane >> 4, lane & 15
                for jb in range(8):
                    s = 16 * g + 2 * jb + i // 8
                    key, col = lds[src[s] + i % 8]
                    t = 8 * rr + jb
                    # A operand (V^T) byte t of lane l: row d = lane % 32 of block c,
                    # the key P's byte t of the same lane holds
                    assert (key, col) == (p_keys_e4m3(lane)[t], 32 * c + lane % 32)

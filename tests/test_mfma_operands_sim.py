"""Host simulation of the matrix-core GEMV's operand layout (k_qgemv_q8_0_mfma).

The kernel sums each q8_0 block with one v_mfma_i32_16x16x32_i8, whose four
k-groups (lanes kq = 0..3 of a column) supply 8 code bytes each.  Which codes a
k-group takes is free as long as weights and activations agree: here k-group kq
takes codes 4kq..4kq+3 and 16+4kq..19+4kq.  Block B's codes are weight dwords
9+kq and 13+kq of the 68-byte pair; block A's sit 2 bytes behind its scale, so
they come from dwords kq, kq+1 and kq+4, kq+5 shifted right by 16 bits.  The
activations sit in LDS per wave: token t's pieces rotated to 16-byte slot
(4p + q + t) % 32.  This test replays, in numpy:

* the byte selection, checking that the four k-groups' operands rebuild each
  block's exact integer sum (and that they partition the block's 32 codes);
* the LDS addresses of the weight reads (rows 272 bytes apart in the ring) and
  of the activation reads, checking that each read puts the 64 lanes on 64
  distinct banks (or, for the per-row scale read, its 16 addresses on 16);
* the staging stores' mapping, checking that every (token, pair, piece) lands
  where the reads look for it.

The GPU tests check the kernel itself against the narrow kernels bitwise."""
import numpy as np

LANES = np.arange(64)
COL = LANES & 15
KQ = LANES >> 4


def _dwords(b):
    return np.frombuffer(np.ascontiguousarray(b, dtype=np.uint8).tobytes(), dtype="<u4")


def _bytes(words):
    return np.frombuffer(np.asarray(words, dtype="<u4").tobytes(), dtype=np.int8)


def _alignbit16(hi, lo):
    return ((int(lo) >> 16) | (int(hi) << 16)) & 0xFFFFFFFF


def _pair(rng):
    ca = rng.integers(-127, 128, 32).astype(np.int8)
    cb = rng.integers(-127, 128, 32).astype(np.int8)
    sa = rng.integers(0, 1 << 16, 2).astype(np.uint8)  # two scale bytes each
    sb = rng.integers(0, 1 << 16, 2).astype(np.uint8)
    pair = np.concatenate([sa, ca.view(np.uint8), sb, cb.view(np.uint8)])
    assert pair.size == 68
    return pair, ca, cb


def test_k_groups_rebuild_each_block_sum():
    rng = np.random.default_rng(7)
    for _ in range(200):
        pair, ca, cb = _pair(rng)
        d = _dwords(pair)  # 17 dwords
        xa = rng.integers(-127, 128, 32).astype(np.int8)
        xb = rng.integers(-127, 128, 32).astype(np.int8)
        a, b = _dwords(xa.view(np.uint8)), _dwords(xb.view(np.uint8))
        sum_a = sum_b = 0
        codes_a, codes_b = [], []
        for kq in range(4):
            wa = _bytes([_alignbit16(d[kq + 1], d[kq]), _alignbit16(d[kq + 5], d[kq + 4])])
            ta = _bytes([a[kq], a[kq + 4]])
            wb = _bytes([d[9 + kq], d[13 + kq]])
            tb = _bytes([b[kq], b[kq + 4]])
            sum_a += int(np.dot(wa.astype(np.int64), ta.astype(np.int64)))
            sum_b += int(np.dot(wb.astype(np.int64), tb.astype(np.int64)))
            idx = list(range(4 * kq, 4 * kq + 4)) + list(range(16 + 4 * kq, 20 + 4 * kq))
            # the weight bytes are the codes of the same indices as the activation bytes
            assert np.array_equal(wa, ca[idx]) and np.array_equal(ta, xa[idx])
            assert np.array_equal(wb, cb[idx]) and np.array_equal(tb, xb[idx])
            codes_a += idx
            codes_b += idx
        assert sorted(codes_a) == list(range(32)) and sorted(codes_b) == list(range(32))
        assert sum_a == int(np.dot(ca.astype(np.int64), xa.astype(np.int64)))
        assert sum_b == int(np.dot(cb.astype(np.int64), xb.astype(np.int64)))


def _distinct_banks(dword_addr):
    return len(set(int(x) % 64 for x in dword_addr)) == len(dword_addr)


def test_ring_reads_hit_distinct_banks():
    row_dw = 272 // 4
    for jj in range(4):
        base = row_dw * COL + 17 * jj
        for off in (0, 1, 4, 5, 9, 13):   # the per-k-group reads (read2 pairs (0,1) (4,5) (9,13))
            assert _distinct_banks(base + KQ + off), (jj, off)
        for off in (0, 8):                # the pair's scale dwords: one address per row
            addrs = sorted(set(int(x) for x in base + off))
            assert len(addrs) == 16 and _distinct_banks(np.array(addrs)), (jj, off)


def test_activation_stage_layout():
    # stores: code load i, lane l moves token t = 2i + l // 32, slot s = l % 32,
    # which holds piece ((s - t) % 32) (pair = that // 4, piece = that % 4)
    where = {}
    for i in range(8):
        for l in range(64):
            t = 2 * i + (l >> 5)
            s = l & 31
            v = (s - t) % 32
            where[(t, v >> 2, v & 3)] = 1024 * i + 16 * l  # byte offset in the wave's stage
    assert len(where) == 16 * 8 * 4
    # reads: lane (token col, kq) takes dword kq of piece q of pair j at
    # 512 col + 16 ((4j + q + col) % 32) + 4 kq
    for j in range(8):
        for q in range(4):
            addr = 512 * COL + 16 * ((4 * j + q + COL) % 32) + 4 * KQ
            for lane in range(64):
                assert addr[lane] == where[(int(COL[lane]), j, q)] + 4 * int(KQ[lane])
            assert _distinct_banks(addr // 4), (j, q)
    # scales: lane l of the scale load moves blocks 4 (l % 4) .. +3 of token
    # l // 4 to floats 4l .. 4l + 3; lane (col, kq) reads blocks 2j, 2j + 1 of
    # token 4kq + r at 16 (4kq + r) + 2j
    lane_of = {}
    for l in range(64):
        for e in range(4):
            lane_of[(l >> 2, 4 * (l & 3) + e)] = 4 * l + e
    for r in range(4):
        for j in range(8):
            for blk in (2 * j, 2 * j + 1):
                assert lane_of[(4 * 0 + r, blk)] == 16 * r + blk
                assert all(lane_of[(4 * kq + r, blk)] == 16 * (4 * kq + r) + blk for kq in range(4))

"""Pins of the oracle's Q4_K and Q6_K decoders.

The pages only name these two formats, so the oracle reads them as the GGUF
k-quant blocks and its parity is UNPINNED with respect to the pages: what is
pinned here is the decoders' arithmetic and bit bookkeeping against that
reading -- every stored bit reaches exactly one (element, bit weight) or one
(scale / min field, bit), the sub-block index of each scale, the value
formulas by brute force over all codes, scales and mins at unit d, and that
each value is the exactly computed formula rounded once to fp32.
"""
import numpy as np

import oracle
import synth


def _f16(v):
    return np.array([v], np.float16).view(np.uint8)


# ------------------------------------------------------------------- Q4_K

def _q4k_block(d=1.0, dmin=1.0, packed=None, codes=None):
    b = np.zeros(synth.Q4_K_BYTES, np.uint8)
    b[0:2] = _f16(d)
    b[2:4] = _f16(dmin)
    if packed is not None:
        b[4:16] = packed
    if codes is not None:
        b[16:144] = codes
    return b


def test_q4_k_block_size():
    assert synth.Q4_K_BYTES == 2 + 2 + 12 + 128
    W = synth.q4_k(np.random.default_rng(0), 1, 3, 512)
    assert W.blocks.shape == (1, 3, 2, 144)
    assert oracle.dequant(W).shape == (1, 3, 512)


def test_q4_k_scale_min_bits_one_to_one():
    """Each of the 96 packed bits sets exactly one bit of one of the 16
    six-bit fields, and every field bit is reached once."""
    seen = set()
    for byte in range(12):
        for bit in range(8):
            p = np.zeros(12, np.uint8)
            p[byte] = 1 << bit
            sc, mn = oracle.q4_k_scales_mins(p)
            f = np.concatenate([sc, mn]).astype(int)
            nz = np.nonzero(f)[0]
            assert len(nz) == 1, (byte, bit, f)
            v = int(f[nz[0]])
            assert v & (v - 1) == 0 and v < 64
            seen.add((int(nz[0]), v.bit_length() - 1))
    assert seen == {(field, b) for field in range(16) for b in range(6)}


def test_q4_k_first_four_fields_are_plain_low_bits():
    p = np.array([5, 63, 0, 17, 9, 1, 62, 33, 0, 0, 0, 0], np.uint8)
    sc, mn = oracle.q4_k_scales_mins(p)
    assert list(sc[:4]) == [5, 63, 0, 17] and list(mn[:4]) == [9, 1, 62, 33]
    assert list(sc[4:]) == [0] * 4 and list(mn[4:]) == [0] * 4


def test_q4_k_values_brute_force_unit_scales():
    """All (q, scale, min) in 16 x 64 x 64 with d = dmin = 1: value = scale*q - min."""
    for q in range(16):
        blocks = np.zeros((64, 64, synth.Q4_K_BYTES), np.uint8)
        blocks[..., 0:2] = _f16(1.0)
        blocks[..., 2:4] = _f16(1.0)
        blocks[..., 4] = np.arange(64, dtype=np.uint8)[:, None]       # scale of sub-block 0
        blocks[..., 8] = np.arange(64, dtype=np.uint8)[None, :]       # min of sub-block 0
        blocks[..., 16:48] = q | (q << 4)                             # sub-blocks 0 and 1
        v = oracle.dequant_q4_k(blocks)[..., :32]
        want = np.arange(64)[:, None] * q - np.arange(64)[None, :]
        assert np.array_equal(v, np.broadcast_to(want[..., None], v.shape).astype(np.float32))


def test_q4_k_element_order_one_to_one():
    """With unit scales and zero mins, a one in one code nibble gives a one in
    exactly one element, and all 256 elements are reached."""
    packed = np.zeros(12, np.uint8)
    packed[0:4] = 1
    packed[8:12] = 1      # low nibbles: scales 4-7 = 1; high nibbles (mins 4-7) = 0
    hits = []
    for byte in range(128):
        for nib in range(2):
            codes = np.zeros(128, np.uint8)
            codes[byte] = 1 << (4 * nib)
            v = oracle.dequant_q4_k(_q4k_block(1.0, 0.0, packed, codes))
            nz = np.nonzero(v)[0]
            assert len(nz) == 1 and v[nz[0]] == 1.0
            hits.append(int(nz[0]))
    assert sorted(hits) == list(range(256))


def test_q4_k_sub_block_of_each_element():
    """Scale j + 1 for sub-block j, all codes 1, no mins: element e = e//32 + 1."""
    sc = np.arange(1, 9, dtype=np.uint8)
    packed = np.zeros(12, np.uint8)
    packed[0:4] = sc[0:4]
    packed[8:12] = sc[4:8]
    v = oracle.dequant_q4_k(_q4k_block(1.0, 0.0, packed, np.full(128, 0x11, np.uint8)))
    assert np.array_equal(v, (np.arange(256) // 32 + 1).astype(np.float32))


def test_q4_k_single_rounding():
    """fp32 decode == the exact value of the formula rounded once."""
    W = synth.q4_k(np.random.default_rng(3), 2, 24, 768)
    b = W.blocks.reshape(-1, synth.Q4_K_BYTES)
    d = b[:, 0:2].copy().view(np.float16)[:, 0].astype(np.float64)
    dmin = b[:, 2:4].copy().view(np.float16)[:, 0].astype(np.float64)
    sc, mn = oracle.q4_k_scales_mins(b[:, 4:16])
    e = np.arange(256)
    byte = b[:, 16:144][:, 32 * (e // 64) + e % 32]
    q = np.where(e % 64 < 32, byte & 15, byte >> 4).astype(np.float64)
    exact = d[:, None] * sc[:, e // 32] * q - dmin[:, None] * mn[:, e // 32]
    assert np.array_equal(oracle.dequant_q4_k(b), exact.astype(np.float32))


# ------------------------------------------------------------------- Q6_K

def _q6k_block(d=1.0, ql=None, qh=None, sc=None):
    b = np.zeros(synth.Q6_K_BYTES, np.uint8)
    if ql is not None:
        b[0:128] = ql
    if qh is not None:
        b[128:192] = qh
    b[192:208] = (np.ones(16, np.int8) if sc is None else np.asarray(sc, np.int8)).view(np.uint8)
    b[208:210] = _f16(d)
    return b


def test_q6_k_block_size():
    assert synth.Q6_K_BYTES == 128 + 64 + 16 + 2
    W = synth.q6_k(np.random.default_rng(0), 1, 3, 512)
    assert W.blocks.shape == (1, 3, 2, 210)
    assert oracle.dequant(W).shape == (1, 3, 512)


def test_q6_k_code_bits_one_to_one():
    """From all-zero codes (every value -32 at unit scales), each of the 1536
    stored code bits raises exactly one element by one power of two; every
    (element, bit weight 1 .. 32) pair is reached once."""
    base = oracle.dequant_q6_k(_q6k_block())
    assert np.all(base == -32.0)
    seen = set()
    for arr, nbytes in (("ql", 128), ("qh", 64)):
        for byte in range(nbytes):
            for bit in range(8):
                x = np.zeros(nbytes, np.uint8)
                x[byte] = 1 << bit
                v = oracle.dequant_q6_k(_q6k_block(ql=x) if arr == "ql" else _q6k_block(qh=x)) - base
                nz = np.nonzero(v)[0]
                assert len(nz) == 1, (arr, byte, bit)
                w = int(v[nz[0]])
                assert w in (1, 2, 4, 8, 16, 32)
                assert (w < 16) == (arr == "ql")
                seen.add((int(nz[0]), w))
    assert seen == {(e, 1 << b) for e in range(256) for b in range(6)}


def test_q6_k_scale_of_each_element():
    """Codes 33 (value 1) everywhere and scale s + 1 (then -(s + 1)) for
    sub-block s: element e = +-(e//16 + 1)."""
    ql = np.full(128, 0x11, np.uint8)   # low 4 bits 1 in both nibbles
    qh = np.full(64, 0xAA, np.uint8)    # top 2 bits 2 at every position: q = 1 + 32
    sc = np.arange(1, 17)
    assert np.array_equal(oracle.dequant_q6_k(_q6k_block(1.0, ql, qh, sc)), (np.arange(256) // 16 + 1).astype(np.float32))
    assert np.array_equal(oracle.dequant_q6_k(_q6k_block(1.0, ql, qh, -sc)), -(np.arange(256) // 16 + 1).astype(np.float32))


def test_q6_k_values_brute_force_unit_d():
    """Every code q in 0..63 with every scale in -128..127 and d = 1:
    value = scale * (q - 32)."""
    sc = np.arange(-128, 128)
    for q in range(64):
        blocks = np.zeros((256, synth.Q6_K_BYTES), np.uint8)
        blocks[:, 0:128] = (q & 15) | ((q & 15) << 4)
        c = q >> 4
        blocks[:, 128:192] = c | (c << 2) | (c << 4) | (c << 6)
        blocks[:, 192:208] = sc.astype(np.int8).view(np.uint8)[:, None]
        blocks[:, 208:210] = _f16(1.0)
        v = oracle.dequant_q6_k(blocks)
        assert np.array_equal(v, np.broadcast_to((sc * (q - 32))[:, None], v.shape).astype(np.float32))


def test_q6_k_single_rounding():
    """fp32 decode == the exact value of the formula rounded once."""
    W = synth.q6_k(np.random.default_rng(4), 2, 24, 768)
    b = W.blocks.reshape(-1, synth.Q6_K_BYTES)
    ql, qh = b[:, 0:128], b[:, 128:192]
    sc = b[:, 192:208].copy().view(np.int8).astype(np.float64)
    d = b[:, 208:210].copy().view(np.float16)[:, 0].astype(np.float64)
    e = np.arange(256)
    n, p, l = e // 128, (e % 128) // 32, e % 32
    lo = ql[:, 64 * n + 32 * (p % 2) + l]
    lo = np.where(p < 2, lo & 15, lo >> 4)
    hi = (qh[:, 32 * n + l] >> (2 * p).astype(np.uint8)) & 3
    q = (lo | (hi << 4)).astype(np.float64) - 32
    exact = d[:, None] * sc[:, e // 16] * q
    assert np.array_equal(oracle.dequant_q6_k(b), exact.astype(np.float32))


def test_spot_positions_of_the_reading():
    """A few positions the reading states outright (so a different but
    still one-to-one order would fail): Q4_K code byte 0 low / high nibble
    -> elements 0 / 32, byte 32 low -> 64, byte 127 high -> 255; Q6_K first
    array byte 0 low / high nibble -> elements 0 / 64, byte 32 low -> 32,
    byte 64 low -> 128; second array byte 0 bits 2-3 -> element 32."""
    packed = np.zeros(12, np.uint8)
    packed[0:4] = 1
    packed[8:12] = 1
    for byte, nib, elem in ((0, 0, 0), (0, 1, 32), (32, 0, 64), (127, 1, 255)):
        codes = np.zeros(128, np.uint8)
        codes[byte] = 1 << (4 * nib)
        assert np.nonzero(oracle.dequant_q4_k(_q4k_block(1.0, 0.0, packed, codes)))[0].tolist() == [elem]
    base = oracle.dequant_q6_k(_q6k_block())
    for byte, shift, elem in ((0, 0, 0), (0, 4, 64), (32, 0, 32), (64, 0, 128)):
        ql = np.zeros(128, np.uint8)
        ql[byte] = 1 << shift
        assert np.nonzero(oracle.dequant_q6_k(_q6k_block(ql=ql)) - base)[0].tolist() == [elem]
    qh = np.zeros(64, np.uint8)
    qh[0] = 1 << 2
    assert np.nonzero(oracle.dequant_q6_k(_q6k_block(qh=qh)) - base)[0].tolist() == [32]

"""Pins for the oracle's block decoders (CPU only).

Each test checks the oracle against something other than its own formula:
hand-built blocks whose decoded values follow from the format description on
the GGUF block-dequant page ("Kernels" items 1-3 and the IQ2_XXS sign-fix
commit), inverse maps written independently of the decoder, round-trip bounds
of an independent quantiser, exact special values and invariants.
"""
import struct

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def h16(x):
    return struct.unpack("<H", np.float16(x).tobytes())[0]


# --------------------------------------------------------------------- Q8_0

def q8_block(d_bits, codes):
    return np.frombuffer(struct.pack("<H", d_bits) + bytes(c & 0xFF for c in codes), np.uint8)


def test_q8_0_block_size_and_signed_codes():
    # scale 0.5; codes cover the whole signed byte range, including 0x80.
    codes = list(range(-128, -96))
    v = oracle.dequant_q8_0(q8_block(h16(0.5), codes)[None])[0]
    assert v.shape == (32,)
    assert np.array_equal(v, np.array(codes, np.float32) * 0.5)
    assert v[0] == -64.0  # byte 0x80 is -128


def test_q8_0_special_scales():
    codes = [1, -1, 127, -127] + [0] * 28
    tiny = oracle.dequant_q8_0(q8_block(0x0001, codes)[None])[0]       # 2**-24
    assert tiny[2] == np.float32(127 * 2.0 ** -24) and tiny[3] == -np.float32(127 * 2.0 ** -24)
    z = oracle.dequant_q8_0(q8_block(0x0000, codes)[None])[0]
    assert np.all(z == 0) and np.signbit(z[1]) and not np.signbit(z[0])
    nan = oracle.dequant_q8_0(q8_block(0x7E00, codes)[None])[0]
    assert np.all(np.isnan(nan))
    inf = oracle.dequant_q8_0(q8_block(0x7C00, codes)[None])[0]
    assert inf[0] == np.inf and inf[1] == -np.inf and np.isnan(inf[4])


def test_q8_0_round_trip_bound():
    # Independent quantiser: d = fp16(amax/127), q = clamp(round(x/d)).
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 32)).astype(np.float32) * 0.3
    blocks = []
    for row in x:
        d = np.float16(np.abs(row).max() / 127)
        q = np.clip(np.rint(row / np.float32(d)), -127, 127).astype(int)
        blocks.append(q8_block(h16(d), q))
    v = oracle.dequant_q8_0(np.stack(blocks))
    d = np.array([np.float16(np.abs(r).max() / 127) for r in x], np.float32)
    bound = d / 2 + np.abs(np.abs(x).max(1) - 127 * d) + 1e-7
    assert np.all(np.abs(v - x) <= bound[:, None])


# --------------------------------------------------------------------- Q2_K

def q2k_block(sc, codes, d_bits, dmin_bits):
    assert len(sc) == 16 and len(codes) == 64
    return np.frombuffer(bytes(sc) + bytes(codes) + struct.pack("<HH", d_bits, dmin_bits), np.uint8)


def test_q2_k_size_is_84():
    assert synth.Q2_K_BYTES == 16 + 64 + 2 + 2 == 84
    v = oracle.dequant_q2_k(q2k_block([0] * 16, [0] * 64, 0, 0)[None])
    assert v.shape == (1, 256)


def test_q2_k_all_scale_min_code_triples():
    # d = dmin = 1: every (q, a, m) must give a*q - m exactly.
    one = h16(1.0)
    for a in range(16):
        for m in range(16):
            sc = [(m << 4) | a] * 16
            for q in range(4):
                codes = [q | (q << 2) | (q << 4) | (q << 6)] * 64
                v = oracle.dequant_q2_k(q2k_block(sc, codes, one, one)[None])[0]
                assert np.all(v == a * q - m), (a, m, q)


def test_q2_k_element_order_one_hot():
    # Inverse map written from the byte/bit side: code byte b, bit pair at 2*s
    # holds element 128*(b//32) + 32*s + b%32.
    one = h16(1.0)
    sc = [1] * 16  # a = 1, m = 0
    for b in range(64):
        for s in range(4):
            codes = [0] * 64
            codes[b] = 1 << (2 * s)
            v = oracle.dequant_q2_k(q2k_block(sc, codes, one, one)[None])[0]
            e = 128 * (b // 32) + 32 * s + b % 32
            expect = np.zeros(256, np.float32)
            expect[e] = 1.0
            assert np.array_equal(v, expect), (b, s)


def test_q2_k_sub_block_scales_are_local():
    one = h16(1.0)
    codes = [0xFF] * 64  # q = 3 everywhere
    for s in range(16):
        sc = [0] * 16
        sc[s] = 0x21  # a = 1, m = 2
        v = oracle.dequant_q2_k(q2k_block(sc, codes, one, one)[None])[0]
        expect = np.zeros(256, np.float32)
        expect[16 * s:16 * s + 16] = 3 * 1 - 2
        assert np.array_equal(v, expect)


def test_q2_k_two_level_scale_values():
    # d = 0.25, dmin = 2: a=3, m=5, q=2 -> 0.25*3*2 - 2*5 = -8.5
    codes = [0xAA] * 64
    v = oracle.dequant_q2_k(q2k_block([0x53] * 16, codes, h16(0.25), h16(2.0))[None])[0]
    assert np.all(v == -8.5)


# ------------------------------------------------------------------ IQ2_XXS

def test_iq2_signs_even_parity_table():
    t = oracle.iq2_signs()
    assert t.shape == (128,) and t.dtype == np.uint8
    for i in range(128):
        assert t[i] & 0x7F == i
        assert bin(int(t[i])).count("1") % 2 == 0
    assert list(t[:8]) == [0, 129, 130, 3, 132, 5, 6, 135]


def iq2_block(d_bits, groups):
    """groups: 8 tuples (idx[4], signs[4] (7-bit), scale nibble)."""
    raw = struct.pack("<H", d_bits)
    for idx, sg, s in groups:
        aux = sg[0] | (sg[1] << 7) | (sg[2] << 14) | (sg[3] << 21) | (s << 28)
        raw += bytes(idx) + struct.pack("<I", aux)
    return np.frombuffer(raw, np.uint8)


def _grid():
    g = np.zeros((256, 8), np.uint8)
    for r in range(256):
        g[r] = [(r * 8 + c) % 251 + 1 for c in range(8)]  # distinct positive rows
    return g


def test_iq2_xxs_grid_rows_and_octets():
    grid = _grid()
    zero = ([0, 0, 0, 0], [0, 0, 0, 0], 1)
    for g in range(8):
        for j in range(4):
            groups = [zero] * 8
            idx = [0, 0, 0, 0]
            idx[j] = 77
            groups[g] = (idx, [0, 0, 0, 0], 1)
            v = oracle.dequant_iq2_xxs(iq2_block(h16(4.0), groups)[None], grid)[0]
            # d=4, s=1 -> group scale 4*(1.5)/4 = 1.5
            expect = np.repeat(grid[0][None], 32, 0).reshape(-1).astype(np.float32) * 1.5
            expect = np.tile(grid[0], 32).astype(np.float32) * 1.5
            expect[32 * g + 8 * j: 32 * g + 8 * j + 8] = grid[77].astype(np.float32) * 1.5
            assert np.array_equal(v, expect), (g, j)


def test_iq2_xxs_sign_bits_one_hot():
    grid = np.full((256, 8), 8, np.uint8)
    for j in range(4):
        for l in range(7):
            sg = [0, 0, 0, 0]
            sg[j] = 1 << l
            groups = [([0] * 4, sg, 0)] + [([0] * 4, [0] * 4, 0)] * 7
            v = oracle.dequant_iq2_xxs(iq2_block(h16(1.0), groups)[None], grid)[0]
            # one stored sign bit -> odd count -> the 8th sign is set too
            neg = {8 * j + l, 8 * j + 7}
            for i in range(256):
                want = -1.0 if i in neg else 1.0
                assert v[i] == want * 8 * 0.125, (j, l, i)


def test_iq2_xxs_even_negatives_per_octet():
    rng = np.random.default_rng(3)
    W = synth.iq2_xxs(rng, 2, 5, 512)
    v = oracle.dequant(W).reshape(-1, 8)
    assert np.all(np.abs(v) > 0)
    assert np.all((v < 0).sum(1) % 2 == 0)


def test_iq2_xxs_scale_nibble_is_per_group_and_monotone():
    grid = np.full((256, 8), 25, np.uint8)
    prev = 0.0
    for s in range(16):
        groups = [([0] * 4, [0] * 4, 0)] * 8
        groups = list(groups)
        groups[3] = ([0] * 4, [0] * 4, s)
        v = oracle.dequant_iq2_xxs(iq2_block(h16(1.0), groups)[None], grid)[0]
        assert np.all(v[96:128] == v[96]) and v[96] > prev
        assert np.all(np.delete(v, np.arange(96, 128)) == v[0])
        prev = v[96]
    assert prev / oracle.dequant_iq2_xxs(iq2_block(h16(1.0), [([0] * 4, [0] * 4, 0)] * 8)[None], grid)[0][0] == 31


# --------------------------------------------------------------------- int4

def test_int4_round_trip_bound():
    rng = np.random.default_rng(11)
    K, G = 256, 64
    x = rng.standard_normal((7, K)).astype(np.float32)
    q = np.zeros((7, K), np.int64)
    s16 = np.zeros((7, K // G), np.float16)
    b16 = np.zeros((7, K // G), np.float16)
    for r in range(7):
        for g in range(K // G):
            seg = x[r, g * G:(g + 1) * G]
            s16[r, g] = np.float16((seg.max() - seg.min()) / 15)
            b16[r, g] = np.float16(seg.min())
            q[r, g * G:(g + 1) * G] = np.clip(np.rint((seg - np.float32(b16[r, g])) / np.float32(s16[r, g])), 0, 15)
    # pack: element 8w+i at bits 4i
    words = np.zeros((7, K // 8), np.uint64)
    for i in range(8):
        words |= (q[:, i::8].astype(np.uint64) << np.uint64(4 * i))
    v = oracle.dequant_int4(words.astype(np.uint32), s16.view(np.uint16), b16.view(np.uint16), G)
    s = np.repeat(s16.astype(np.float32), G, 1)
    slack = np.repeat(np.abs(b16.astype(np.float32) - x.reshape(7, K // G, G).min(2)), G, 1) + 16 * 1e-3 * s
    assert np.all(np.abs(v - x) <= s / 2 + slack + 1e-6)


def test_int4_nibble_positions():
    one = np.array([[h16(1.0)]], np.uint16)
    zero = np.array([[0]], np.uint16)
    for i in range(8):
        words = np.zeros((1, 8), np.uint32)
        words[0, 3] = 0x9 << (4 * i)
        v = oracle.dequant_int4(words, one, zero, 64)[0]
        expect = np.zeros(64, np.float32)
        expect[8 * 3 + i] = 9
        assert np.array_equal(v, expect)


def test_int4_pick_expert_from_stack():
    # Four stacked experts; expert 2's slab decodes like the lone tensor.
    rng = np.random.default_rng(2)
    W = synth.int4(rng, 4, 6, 128)
    lone = synth.QWeights("int4", 1, 6, 128, 64, qs=W.qs[2:3], scale=W.scale[2:3], bias=W.bias[2:3])
    assert np.array_equal(oracle.dequant(W)[2], oracle.dequant(lone)[0])
    assert not np.array_equal(oracle.dequant(W)[1], oracle.dequant(lone)[0])


# ------------------------------------------------------------- output roundings

def test_round_bf16_ties_and_specials():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.0, 0.0, -0.0, np.inf, 1 + 2 ** -7], np.float32)
    got = oracle.round_bf16(vals)
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000, 0x8000, 0x7F80, 0x3F81]
    n = oracle.round_bf16(np.array([np.nan], np.float32))[0]
    assert (n & 0x7F80) == 0x7F80 and (n & 0x7F) != 0


def test_round_f16_subnormal_and_tie():
    got = oracle.round_f16(np.array([2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 1 + 2 ** -11], np.float32))
    assert list(got) == [0x0001, 0x0000, 0x0002, 0x3C00]


# ------------------------------------------------------------ golden layouts

def _golden_layouts():
    import os
    rows = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", "block_layouts.txt")):
        if line.strip() and not line.startswith("#"):
            key, *vals = line.split()
            rows[key] = [int(v) for v in vals]
    return rows


def test_golden_block_layouts():
    """tests/golden/block_layouts.txt: block sizes and first code byte (the
    Q2_K row and the grid size as the pages state them, the Q8_0 and IQ2_XXS
    byte positions as readings c1 / c3); a code planted at that byte decodes
    into element 0."""
    g = _golden_layouts()
    rng = np.random.default_rng(0)
    # Q8_0: fp16 scale 1.0, code 5 at the first code byte -> element 0 == 5
    vals, nbytes, first = g["q8_0"]
    blk = np.zeros((1, nbytes), np.uint8)
    blk[0, 0:2] = np.frombuffer(struct.pack("<H", h16(1.0)), np.uint8)
    blk[0, first] = 5
    v = oracle.dequant_q8_0(blk)
    assert v.shape[-1] == vals and v.reshape(-1)[0] == 5.0 and np.all(v.reshape(-1)[1:] == 0)
    assert synth.q8_0(rng, 1, 1, vals).blocks.shape[-1] == nbytes
    # Q2_K: every sub-block scale 1 / min 0, d = 1, dmin = 0, code 3 in the
    # low 2 bits of the first code byte -> element 0 == 3, all others 0
    vals, nbytes, first = g["q2_k"]
    blk = np.zeros((1, nbytes), np.uint8)
    blk[0, 0:16] = 0x01
    blk[0, first] = 0x03
    blk[0, nbytes - 4:nbytes - 2] = np.frombuffer(struct.pack("<H", h16(1.0)), np.uint8)
    v = oracle.dequant_q2_k(blk).reshape(-1)
    assert v.size == vals and v[0] == 3.0 and np.all(v[1:] == 0)
    assert synth.q2_k(rng, 1, 1, vals).blocks.shape[-1] == nbytes
    # IQ2_XXS: d = 8 and scale nibble 0 give group scale 1; grid index 1 in
    # the first code byte, no signs -> elements 0..7 == grid row 1
    vals, nbytes, first = g["iq2_xxs"]
    rows, per_row, total = g["grid"]
    grid = synth.iq2_grid()
    assert grid.size == total and grid.shape == (rows, per_row)
    blk = np.zeros((1, nbytes), np.uint8)
    blk[0, 0:2] = np.frombuffer(struct.pack("<H", h16(8.0)), np.uint8)
    blk[0, first] = 1
    v = oracle.dequant_iq2_xxs(blk, grid).reshape(-1)
    assert v.size == vals
    assert np.array_equal(v[:8], grid[1].astype(np.float32))
    assert np.array_equal(v[8:32], np.repeat(grid[0].astype(np.float32)[None], 3, 0).reshape(-1))
    assert synth.iq2_xxs(rng, 1, 1, vals).blocks.shape[-1] == nbytes

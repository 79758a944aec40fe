"""Pins of the oracle's MXFP4 decoding (no GPU): the page's value table and
block layout, closed forms of the scale, and brute force on every code."""
import os

import numpy as np

import oracle
import synth


def _golden(name):
    rows = {}
    for line in open(os.path.join(os.path.dirname(__file__), "golden", name)):
        if line.strip() and not line.startswith("#"):
            key, *vals = line.split()
            rows[key] = vals
    return rows


G = _golden("mxfp4_table.txt")


def test_value_table_matches_the_page():
    # codes 0-7 are the table's magnitudes in order, codes 8-15 their negatives
    mags = [float(v) for v in G["magnitudes"]]
    vals = oracle.e2m1_value(np.arange(16))
    assert vals[:8].tolist() == mags
    assert vals[8:].tolist() == [-m for m in mags]
    assert np.isfinite(vals).all()  # no NaN among the 16 codes


def test_scale_closed_forms():
    assert oracle.e8m0_scale(127) == 1.0
    assert oracle.e8m0_scale(128) == 2.0 and oracle.e8m0_scale(120) == 2.0 ** -7
    assert oracle.e8m0_scale(0) == 2.0 ** -127 and oracle.e8m0_scale(254) == 2.0 ** 127
    assert np.isnan(oracle.e8m0_scale(int(G["nan_exponent"][0])))


def test_block_layout_low_nibble_first():
    # a hand-built block: e = 127 + 1 (scale 2); code byte i = (hi << 4) | lo
    # holds elements 2i (lo) and 2i + 1 (hi)
    blk = np.zeros(int(G["block_bytes"][0]), np.uint8)
    blk[0] = 128
    blk[1] = 0x31   # elements 0, 1: codes 1 (0.5), 3 (1.5)
    blk[2] = 0xF7   # elements 2, 3: codes 7 (6.0), 15 (-6.0)
    blk[16] = 0x9A  # elements 30, 31: codes 10 (-1.0), 9 (-0.5)
    v = oracle.dequant_mxfp4(blk[None])[0]
    assert v.shape == (int(G["block_values"][0]),)
    assert v[:4].tolist() == [1.0, 3.0, 12.0, -12.0]
    assert v[30:].tolist() == [-2.0, -1.0]
    assert (v[4:30] == 0).all()


def test_every_code_every_scale_brute_force():
    # all 16 codes at several exponents against the table times 2^(e-127),
    # including the subnormal-scale end and the NaN sentinel
    mags = [float(x) for x in G["magnitudes"]]
    table = mags + [-m for m in mags]
    for e in (0, 1, 100, 127, 200, 254, 255):
        blk = np.zeros((2, 17), np.uint8)
        blk[:, 0] = e
        codes = np.arange(32) % 16
        pairs = codes.reshape(16, 2)
        blk[:, 1:] = (pairs[:, 0] | (pairs[:, 1] << 4)).astype(np.uint8)
        v = oracle.dequant_mxfp4(blk)
        if e == 255:
            assert np.isnan(v).all()
            continue
        expect = np.array([table[c] * 2.0 ** (e - 127) for c in codes], np.float64)
        with np.errstate(over="ignore"):  # e = 254: |value| >= 2 is past fp32's range
            assert np.array_equal(v[0], expect.astype(np.float32))
        if e == 254:
            assert np.isinf(v[0][[4, 5, 6, 7]]).all() and v[0][3] == np.float32(1.5 * 2.0 ** 127)
        assert np.array_equal(v[1], v[0])


def test_qmm_on_mxfp4_is_dequant_then_matmul():
    rng = np.random.default_rng(3)
    W = synth.mxfp4(rng, 2, 16, 128)
    x = rng.standard_normal((5, 128))
    full = oracle.dequant(W).astype(np.float64)
    assert np.allclose(oracle.qmm(x, W, e=1), x @ full[1].T, rtol=1e-13, atol=1e-13)

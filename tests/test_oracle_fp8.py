"""Pins of the oracle's FP8 E4M3 block decoding (no GPU): the page's format
parameters, closed forms, brute force over all 256 bytes, and the page's
reference quantizer round trip."""
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


G = _golden("fp8_e4m3.txt")


def test_format_parameters():
    v = oracle.e4m3_value(np.arange(256))
    nan = [int(b) for b in G["nan_bytes"]]
    assert np.isnan(v[nan]).all() and np.isfinite(np.delete(v, nan)).all()
    assert np.nanmax(v) == float(G["max_value"][0]) and np.nanmin(v) == -float(G["max_value"][0])
    bias = int(G["bias"][0])
    assert oracle.e4m3_value(bias << 3) == 1.0          # exponent field = bias, mantissa 0
    assert oracle.e4m3_value(0x01) == 2.0 ** (-6 - 3)   # smallest subnormal
    assert oracle.e4m3_value(0x08) == 2.0 ** -6         # smallest normal
    assert oracle.e4m3_value(0x80) == 0.0 and np.signbit(oracle.e4m3_value(0x80))


def test_all_bytes_brute_force():
    # every byte against sign * 2^(E - bias) * (1 + m / 8) (E > 0) or
    # sign * 2^(1 - bias) * m / 8 (E = 0), written with integers
    for b in range(256):
        if b & 0x7F == 0x7F:
            continue
        s, E, m = b >> 7, (b >> 3) & 15, b & 7
        mag = (8 + m) * 2.0 ** (E - 7 - 3) if E else m * 2.0 ** (1 - 7 - 3)
        assert oracle.e4m3_value(b) == (-mag if s else mag), b
    # positive codes are increasing
    pos = oracle.e4m3_value(np.arange(0x7F))
    assert (np.diff(pos) > 0).all()


def test_block_scales_and_layout():
    W = synth.fp8(np.random.default_rng(0), 1, 256, 256)
    d = oracle.dequant(W)[0]
    v = oracle.e4m3_value(W.qs[0]).astype(np.float32)
    for (i, j) in [(0, 0), (127, 127), (128, 0), (5, 200), (255, 255)]:
        assert d[i, j] == np.float32(v[i, j] * W.scale[0, i // 128, j // 128])
    # row selection views use one scale row per weight row
    rows = np.array([3, 130, 255])
    assert np.array_equal(oracle.dequant_rows(W, 0, rows), d[rows])


def test_reference_quantizer_round_trip():
    # the page's quantizer: scale = max|w| / 448 per block, nearest byte
    rng = np.random.default_rng(1)
    w = rng.standard_normal((128, 256)) * 0.05
    finite = np.array([b for b in range(256) if b & 0x7F != 0x7F])
    vals = oracle.e4m3_value(finite)
    scales = np.stack([np.abs(w[:, 0:128]).max(), np.abs(w[:, 128:]).max()]) / 448.0
    q = np.empty(w.shape, np.uint8)
    for j in range(2):
        blk = w[:, 128 * j:128 * (j + 1)] / scales[j]
        q[:, 128 * j:128 * (j + 1)] = finite[np.abs(blk[..., None] - vals).argmin(-1)]
    back = oracle.dequant_fp8_block(q, scales.reshape(1, 2).astype(np.float32))
    # nearest E4M3 value: relative error at most 2^-4 above the subnormal range
    big = np.abs(w) > 2.0 ** -6 * scales.max()
    assert (np.abs(back - w)[big] <= np.abs(w)[big] * 2.0 ** -4 + 1e-9).all()
    assert np.abs(back).max() <= 448 * scales.max() * (1 + 1e-6)


def test_qmm_on_fp8_is_dequant_then_matmul():
    rng = np.random.default_rng(3)
    W = synth.fp8(rng, 2, 128, 256)
    x = rng.standard_normal((5, 256))
    full = oracle.dequant(W).astype(np.float64)
    assert np.allclose(oracle.qmm(x, W, e=1), x @ full[1].T, rtol=1e-13, atol=1e-13)

"""Host-side checks of libqmoe (no GPU): the library loads, exports every
entry point include/qmoe.h declares, the loader split reproduces the on-disk
blocks, and argument validation rejects bad calls before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "qmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = qm.lib()
    names = _declared()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(qm.EXPORTS)


def test_split_q8_0_tiled_layout():
    """Every code and scale lands where the header's tiled layout says."""
    rows, k = 32, 192
    W = synth.q8_0(np.random.default_rng(0), 2, rows // 2, k)
    qs, d = qm.split_q8_0(W.blocks, rows, k)
    b = W.blocks.reshape(rows, k // 32, 34)
    q = qs.view(np.uint8).reshape(rows // 16, k // 64, 4, 16, 16)
    d = d.view(np.uint8).reshape(rows // 16, k // 32, 16, 2)
    for R in range(rows):
        for j in range(k // 32):
            assert np.array_equal(d[R // 16, j, R % 16], b[R, j, :2])
            for h in range(2):
                kk = 32 * j + 16 * h
                assert np.array_equal(q[R // 16, kk // 64, (kk % 64) // 16, R % 16], b[R, j, 2 + 16 * h:18 + 16 * h])


def test_split_q2_k_tiled_layout():
    """Every byte of each block lands where the header's tiled layout says."""
    rows, k = 32, 512
    W = synth.q2_k(np.random.default_rng(1), 2, rows // 2, k)
    qs, sc, d, dmin = qm.split_q2_k(W.blocks, rows, k)
    b = W.blocks.reshape(rows, k // 256, 84)
    SB = k // 256
    q8 = qs.view(np.uint8).reshape(rows // 16, SB, 2, 16, 32)
    sc = sc.reshape(rows // 16, SB, 16, 16)
    d = d.view(np.uint8).reshape(rows // 16, SB, 16, 2)
    dmin = dmin.view(np.uint8).reshape(rows // 16, SB, 16, 2)
    for R in range(rows):
        for s_ in range(SB):
            blk = b[R, s_]
            assert np.array_equal(sc[R // 16, s_, R % 16], blk[:16])
            for h in range(2):
                assert np.array_equal(q8[R // 16, s_, h, R % 16], blk[16 + 32 * h:48 + 32 * h])
            assert np.array_equal(d[R // 16, s_, R % 16], blk[80:82])
            assert np.array_equal(dmin[R // 16, s_, R % 16], blk[82:84])
    with pytest.raises(qm.QmoeError):
        qm.split_q2_k(W.blocks[:1], 8, k)   # 8 rows: not a multiple of 16


def test_split_iq2_xxs_tiled_layout():
    rows, k = 16, 768
    W = synth.iq2_xxs(np.random.default_rng(2), 1, rows, k)
    ia, d = qm.split_iq2_xxs(W.blocks, rows, k)
    SB = k // 256
    b = W.blocks.reshape(rows, SB, 66)
    ia = ia.view(np.uint8).reshape(rows // 16, SB, 8, 16, 8)
    d = d.view(np.uint8).reshape(rows // 16, SB, 16, 2)
    for R in range(rows):
        for s_ in range(SB):
            blk = b[R, s_]
            assert np.array_equal(d[R // 16, s_, R % 16], blk[:2])
            for g in range(8):
                assert np.array_equal(ia[R // 16, s_, g, R % 16], blk[2 + 8 * g:10 + 8 * g])


def test_split_mxfp4_tiled_layout():
    """Every code and exponent lands where the header's tiled layout says."""
    rows, k = 32, 192
    W = synth.mxfp4(np.random.default_rng(2), 2, rows // 2, k)
    qs, e = qm.split_mxfp4(W.blocks, rows, k)
    b = W.blocks.reshape(rows, k // 32, 17)
    q = qs.reshape(rows // 16, k // 64, 2, 16, 4)
    e = e.reshape(rows // 16, k // 32, 16)
    for R in range(rows):
        for j in range(k // 32):
            assert e[R // 16, j, R % 16] == b[R, j, 0]
            codes = np.stack([b[R, j, 1:] & 15, b[R, j, 1:] >> 4], 1).reshape(32)  # element order
            for w in range(4):
                word = int(q[R // 16, j // 2, j % 2, R % 16, w])
                for i in range(4):
                    byte = (word >> (8 * i)) & 0xFF
                    assert byte & 15 == codes[8 * w + 2 * i] and byte >> 4 == codes[8 * w + 2 * i + 1]
    with pytest.raises(qm.QmoeError):
        qm.split_mxfp4(W.blocks[:, :8], 8 * 2 // 2, k)


def test_split_q4_k_tiled_layout():
    """Decoding the tiled arrays as the header lays them out gives the
    oracle's values for every element (the oracle reads the on-disk blocks)."""
    rows, k = 32, 512
    W = synth.q4_k(np.random.default_rng(5), 2, rows // 2, k)
    qs, sm, d, dmin = qm.split_q4_k(W.blocks, rows, k)
    SB = k // 256
    qs = qs.reshape(rows // 16, SB, 4, 16, 32)
    sm = sm.reshape(rows // 16, SB, 16, 16)
    d = d.reshape(rows // 16, SB, 16).view(np.float16).astype(np.float32)
    dmin = dmin.reshape(rows // 16, SB, 16).view(np.float16).astype(np.float32)
    e = np.arange(256)
    R = np.arange(rows)
    byte = qs[R[:, None, None] // 16, np.arange(SB)[None, :, None], (e // 64)[None, None, :], R[:, None, None] % 16,
              (e % 32)[None, None, :]]
    q = np.where(e % 64 < 32, byte & 15, byte >> 4).astype(np.float32)
    rb, r, sb = R[:, None, None] // 16, R[:, None, None] % 16, np.arange(SB)[None, :, None]
    sc = sm[rb, sb, r, (e // 32)[None, None, :]].astype(np.float32)
    mn = sm[rb, sb, r, 8 + (e // 32)[None, None, :]].astype(np.float32)
    v = (d[rb, sb, r] * sc) * q - dmin[rb, sb, r] * mn
    assert np.array_equal(v.reshape(rows, k), oracle.dequant(W).reshape(rows, k))
    with pytest.raises(qm.QmoeError):
        qm.split_q4_k(W.blocks[:, :, :1], rows, k)


def test_split_q6_k_tiled_layout():
    rows, k = 32, 512
    W = synth.q6_k(np.random.default_rng(6), 2, rows // 2, k)
    qs, qh, sc, d = qm.split_q6_k(W.blocks, rows, k)
    SB = k // 256
    qs = qs.reshape(rows // 16, SB, 4, 16, 32)
    qh = qh.reshape(rows // 16, SB, 2, 16, 32)
    sc = sc.reshape(rows // 16, SB, 16, 16).astype(np.float32)
    d = d.reshape(rows // 16, SB, 16).view(np.float16).astype(np.float32)
    e = np.arange(256)[None, None, :]
    R = np.arange(rows)
    rb, r, sb = R[:, None, None] // 16, R[:, None, None] % 16, np.arange(SB)[None, :, None]
    lo = qs[rb, sb, e // 64, r, e % 32]
    lo = np.where(e % 64 < 32, lo & 15, lo >> 4)
    hi = (qh[rb, sb, e // 128, r, e % 32] >> (2 * ((e % 128) // 32)).astype(np.uint8)) & 3
    q = (lo | (hi << 4)).astype(np.float32) - 32
    v = (d[rb, sb, r] * sc[rb, sb, r, e // 16]) * q
    assert np.array_equal(v.reshape(rows, k), oracle.dequant(W).reshape(rows, k))
    with pytest.raises(qm.QmoeError):
        qm.split_q6_k(W.blocks[:, :, :1], rows, k)


def test_split_fp8_tiled_layout():
    """Every code lands where the header's tiled layout says (the Q8_0 code tiling)."""
    rows, k = 256, 384
    W = synth.fp8(np.random.default_rng(4), 2, rows // 2, k)
    qs = qm.split_fp8(W.qs, rows, k).reshape(rows // 16, k // 64, 4, 16, 16)
    w = W.qs.reshape(rows, k)
    for R in range(0, rows, 7):
        for kk in range(k):
            assert qs[R // 16, kk // 64, (kk % 64) // 16, R % 16, kk % 16] == w[R, kk]
    with pytest.raises(qm.QmoeError):
        qm.split_fp8(W.qs[:1, :64], 64, k)             # rows not a multiple of 128
    with pytest.raises(qm.QmoeError):
        qm.split_fp8(W.qs[..., :192], rows, 192)      # k not a multiple of 128


def test_split_int4_tiled_layout():
    """Every element of the MLX rows lands where the header's tiled layout says."""
    rng = np.random.default_rng(3)
    rows, k, group = 48, 192, 64
    words = rng.integers(0, 2**32, size=rows * k // 8, dtype=np.uint64).astype(np.uint32)
    scale = rng.integers(0, 2**16, size=rows * k // group, dtype=np.uint64).astype(np.uint16)
    bias = rng.integers(0, 2**16, size=rows * k // group, dtype=np.uint64).astype(np.uint16)
    qs, sb = qm.split_int4(words, scale, bias, rows, k, group)
    mlx = (words.reshape(rows, k // 8, 1) >> (4 * np.arange(8, dtype=np.uint32))) & 15  # element 8w+j -> nibble j
    mlx = mlx.reshape(rows, k)
    for R in range(rows):
        for kk in range(k):
            tile = (R // 16) * (k // 64) + kk // 64
            lane = 16 * ((kk % 64) // 16) + R % 16
            word = int(qs[(tile * 64 + lane) * 2 + (kk % 16) // 8])
            j = kk % 8
            assert (word >> (4 * (j // 2) + 16 * (j % 2))) & 15 == mlx[R, kk]
    for R in range(rows):
        for gi in range(k // group):
            v = int(sb[((R // 16) * (k // group) + gi) * 16 + R % 16])
            assert v & 0xFFFF == scale[R * (k // group) + gi] and v >> 16 == bias[R * (k // group) + gi]


def test_split_int4_rejects_untileable_shapes():
    z = np.zeros(16 * 96 // 8, np.uint32)
    s = np.zeros(16 * 96 // 32, np.uint16)
    with pytest.raises(qm.QmoeError):
        qm.split_int4(z, s, s, 16, 96, 32)          # k not a multiple of 64
    z = np.zeros(16 * 64 // 8, np.uint32)
    s = np.zeros(16 * 64 // 48, np.uint16)
    with pytest.raises(qm.QmoeError):
        qm.split_int4(z, s, s, 16, 64, 48)          # group not 32 / 64 / 128 / 256


def test_signs_table_matches_oracle():
    assert np.array_equal(qm.iq2_signs_table(), oracle.iq2_signs())


def _plan_words(T, k, E):
    P = T * k
    words = 8 + E + E + 1 + P
    words = (words + 3) & ~3
    words += 4 * (min(P, E) + P // 16) + P
    words += ((P + 1023) // 1024) * E  # chunk histogram scratch
    if P >= 2048:  # work-balancing area: 512 tickets and 512 partial tiles of 80 x 256 fp32
        words = (words + 63) & ~63
        words += 512 + 512 * 80 * 256
    return words


def test_plan_bytes_layout():
    assert qm.plan_bytes(2048, 8, 256, 128) == 4 * _plan_words(2048, 8, 256)
    assert qm.plan_bytes(255, 8, 64, 80) == 4 * _plan_words(255, 8, 64)      # P = 2040: no balancing area
    assert qm.plan_bytes(256, 8, 64, 80) == 4 * _plan_words(256, 8, 64)      # P = 2048: with it
    assert qm.plan_bytes(256, 8, 64, 80) - qm.plan_bytes(255, 8, 64, 80) > 40 << 20


def test_argument_validation_before_launch():
    L = qm.lib()
    E = -1
    # plan: topk above 8, experts above 1024, bad bm, NULL ids
    assert L.qmoe_moe_plan(ctypes.c_void_p(16), 4, 9, 8, 80, ctypes.c_void_p(16), 1 << 20, None) == -4
    assert L.qmoe_moe_plan(ctypes.c_void_p(16), 4, 2, 2000, 80, ctypes.c_void_p(16), 1 << 20, None) == -4
    assert L.qmoe_moe_plan(ctypes.c_void_p(16), 4, 2, 8, 40, ctypes.c_void_p(16), 1 << 20, None) == E
    assert L.qmoe_moe_plan(ctypes.c_void_p(16), 4, 2, 8, 144, ctypes.c_void_p(16), 1 << 20, None) == E
    assert L.qmoe_moe_plan(None, 4, 2, 8, 80, ctypes.c_void_p(16), 1 << 20, None) == E
    # plan tiles taller than the matmul's 80-row register tile are refused,
    # so a plan and the matmul always accept the same tile heights
    for bm in (96, 112, 128):
        assert L.qmoe_moe_plan(ctypes.c_void_p(16), 4, 2, 8, bm, ctypes.c_void_p(16), 1 << 20, None) == -2
    # plan buffer too small
    assert L.qmoe_moe_plan(ctypes.c_void_p(16), 4, 2, 8, 80, ctypes.c_void_p(16), 16, None) == -5
    # misaligned plan
    assert L.qmoe_moe_plan(ctypes.c_void_p(16), 4, 2, 8, 80, ctypes.c_void_p(20), 1 << 20, None) == -6
    # dequant: NULL / misaligned / bad dtype
    assert L.qmoe_dequant_q8_0(None, ctypes.c_void_p(16), 16, 64, ctypes.c_void_p(16), 1, None) == E
    assert L.qmoe_dequant_q8_0(ctypes.c_void_p(8), ctypes.c_void_p(16), 16, 64, ctypes.c_void_p(16), 1, None) == -6
    assert L.qmoe_dequant_q8_0(ctypes.c_void_p(16), ctypes.c_void_p(16), 16, 64, ctypes.c_void_p(16), 7, None) == E
    assert L.qmoe_dequant_q8_0(ctypes.c_void_p(16), ctypes.c_void_p(16), 16, 96, ctypes.c_void_p(16), 1, None) == -3
    assert L.qmoe_dequant_int4(ctypes.c_void_p(16), ctypes.c_void_p(16), 16, 96, 32,
                               ctypes.c_void_p(16), 1, None) == -3
    assert L.qmoe_dequant_int4(ctypes.c_void_p(16), ctypes.c_void_p(16), 16, 128, 48,
                               ctypes.c_void_p(16), 1, None) == -3
    # tiled formats: k not a multiple of 256 (any row count is accepted)
    P16 = ctypes.c_void_p(16)
    assert L.qmoe_dequant_q2_k(P16, P16, P16, P16, 8, 320, P16, 1, None) == -3
    assert L.qmoe_dequant_iq2_xxs(P16, P16, P16, P16, 16, 128, P16, 1, None) == -3
    assert L.qmoe_dequant_q4_k(P16, P16, P16, P16, 16, 320, P16, 1, None) == -3
    assert L.qmoe_dequant_q6_k(P16, P16, P16, P16, 16, 512 + 64, P16, 1, None) == -3
    assert L.qmoe_dequant_q4_k(P16, P16, P16, None, 16, 256, P16, 1, None) == E
    assert L.qmoe_dequant_q6_k(P16, None, P16, P16, 16, 256, P16, 1, None) == E
    assert L.qmoe_dequant_q6_k(P16, ctypes.c_void_p(8), P16, P16, 16, 256, P16, 1, None) == -6
    # k-quant weights in a matmul: k a multiple of 256; Q4_K needs d and dmin, Q6_K the top-bit array
    w = qm._Weights(qm.Q4_K, 1, 64, 320, 0, 0, 16, 0, 16, 0, 16, 16, 0, 0)
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 1, 4, 0, ctypes.c_void_p(16), 1, None) == -3
    w = qm._Weights(qm.Q4_K, 1, 64, 256, 0, 0, 16, 0, 16, 0, 16, 0, 0, 0)
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 1, 4, 0, ctypes.c_void_p(16), 1, None) == E
    w = qm._Weights(qm.Q6_K, 1, 64, 256, 0, 0, 16, 0, 16, 0, 16, 0, 0, 0)
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 1, 4, 0, ctypes.c_void_p(16), 1, None) == E
    # FP8: rows and k multiples of the 128 x 128 scale block; scales required
    assert L.qmoe_dequant_fp8(P16, P16, 64, 128, P16, 1, None) == -3
    assert L.qmoe_dequant_fp8(P16, P16, 128, 192, P16, 1, None) == -3
    assert L.qmoe_dequant_fp8(P16, None, 128, 128, P16, 1, None) == E
    w = qm._Weights(qm.FP8, 2, 64, 256, 0, 0, 16, 0, 16, 0, 0, 0, 0, 0)   # n not a multiple of 128
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 1, 4, 0, ctypes.c_void_p(16), 1, None) == -3
    w = qm._Weights(qm.FP8, 1, 128, 256, 0, 0, 16, 0, 0, 0, 0, 0, 0, 0)   # no scales
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 1, 4, 0, ctypes.c_void_p(16), 1, None) == E
    # matmul: k not a block multiple, too many experts, wrong epilogue / dtype
    w = qm._Weights(qm.Q2_K, 1, 64, 320, 0, 0, 16, 0, 16, 0, 16, 16, 0, 0)
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 1, 4, 0, ctypes.c_void_p(16), 1, None) == -3
    w = qm._Weights(qm.Q8_0, 2000, 64, 256, 0, 0, 16, 0, 16, 0, 0, 0, 0, 0)
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 1, 4, 0, ctypes.c_void_p(16), 1, None) == -4
    w = qm._Weights(qm.Q8_0, 1, 64, 256, 0, 0, 16, 0, 16, 0, 0, 0, 0, 0)
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 1, 4, 3, ctypes.c_void_p(16), 1, None) == -2
    assert L.qmoe_qmm_dense(ctypes.byref(w), ctypes.c_void_p(16), 0, 4, 0, ctypes.c_void_p(16), 1, None) == E
    w = qm._Weights(qm.INT4, 4, 64, 256, 32, 0, 16, 0, 16, 16, 0, 0, 0, 0)
    assert L.qmoe_moe_gather_qmm(ctypes.byref(w), ctypes.c_void_p(16), 4, 2, 128, ctypes.c_void_p(16), 2, 0,
                                 None, 0, ctypes.c_void_p(16), 2, None) == -2  # bf16 needs group >= 64
    # gemv: batch above the limit, combine needs weights
    w = qm._Weights(qm.INT4, 4, 64, 512, 64, 0, 16, 0, 16, 16, 0, 0, 0, 0)
    assert L.qmoe_moe_gemv(ctypes.byref(w), ctypes.c_void_p(16), 2, 65, ctypes.c_void_p(16), None, 8, 1,
                           ctypes.c_void_p(16), 2, None) == -4
    assert L.qmoe_moe_gemv(ctypes.byref(w), ctypes.c_void_p(16), 2, 4, ctypes.c_void_p(16), None, 8, 2,
                           ctypes.c_void_p(16), 2, None) == E
    # empty inputs return OK without touching the device
    assert L.qmoe_dequant_q8_0(ctypes.c_void_p(16), ctypes.c_void_p(16), 0, 64, ctypes.c_void_p(16), 1, None) == 0
    assert L.qmoe_moe_gemv(ctypes.byref(w), ctypes.c_void_p(16), 2, 0, ctypes.c_void_p(16), None, 8, 1,
                           ctypes.c_void_p(16), 2, None) == 0
    # router top-k: softmax takes no scale; topk within [1, min(8, E)]
    P = ctypes.c_void_p(16)
    r = L.qmoe_router_topk
    assert r(P, 2, 4, 128, 8, 0, None, 2.0, P, P, None) == E
    assert r(P, 2, 4, 128, 9, 1, None, 1.0, P, P, None) == -4
    assert r(P, 2, 4, 2048, 8, 1, None, 1.0, P, P, None) == -4
    assert r(P, 2, 4, 4, 6, 1, None, 1.0, P, P, None) == E
    assert r(P, 2, 4, 128, 8, 2, None, 1.0, P, P, None) == E
    assert r(P, 5, 4, 128, 8, 1, None, 1.0, P, P, None) == E
    assert r(None, 2, 4, 128, 8, 1, None, 1.0, P, P, None) == E
    assert r(ctypes.c_void_p(17), 2, 4, 128, 8, 1, None, 1.0, P, P, None) == -6
    assert r(P, 0, 4, 128, 8, 1, ctypes.c_void_p(18), 1.0, P, P, None) == -6
    assert r(P, 2, 0, 128, 8, 1, None, 1.0, P, P, None) == 0
    assert qm.lib().qmoe_strerror(-4).decode().startswith("size limit")


def test_no_gpu_means_arch_error():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert qm.lib().qmoe_check_device() == -7


def _with_zero_rows(aos, rows, k, block_vals, block_bytes, pad):
    """On-disk blocks of `rows` rows followed by `pad` rows of zero blocks."""
    a = np.asarray(aos, np.uint8).reshape(rows, k // block_vals, block_bytes)
    return np.concatenate([a, np.zeros((pad, k // block_vals, block_bytes), np.uint8)])


@pytest.mark.parametrize("rows", [1, 5, 20, 33])
def test_split_any_row_count_pads_with_zero_rows(rows):
    """Any row count splits: the tiled arrays are sized for split_rows(rows)
    rows and equal the split of the same matrix with zero rows appended up to
    the next multiple of 16 (so the kernels may read whole 16-row blocks)."""
    R = qm.split_rows(rows)
    assert R % 16 == 0 and rows <= R < rows + 16
    rng = np.random.default_rng(rows)
    k = 512
    for fmt, bv, bb, split in (("q8_0", 32, 34, qm.split_q8_0), ("q2_k", 256, 84, qm.split_q2_k),
                               ("iq2_xxs", 256, 66, qm.split_iq2_xxs), ("mxfp4", 32, 17, qm.split_mxfp4),
                               ("q4_k", 256, 144, qm.split_q4_k), ("q6_k", 256, 210, qm.split_q6_k)):
        W = synth.weights(fmt, rng, 1, rows, k)
        got = split(W.blocks, rows, k)
        ref = split(_with_zero_rows(W.blocks, rows, k, bv, bb, R - rows), R, k)
        for g, r in zip(got, ref):
            assert g.size == r.size and np.array_equal(g, r), fmt
    W = synth.int4(rng, 1, rows, k)

    def pad(a):
        a = a.reshape(rows, -1)
        return np.concatenate([a, np.zeros((R - rows, a.shape[1]), a.dtype)])

    got = qm.split_int4(W.qs, W.scale, W.bias, rows, k, 64)
    ref = qm.split_int4(pad(W.qs), pad(W.scale), pad(W.bias), R, k, 64)
    for g, r in zip(got, ref):
        assert g.size == r.size and np.array_equal(g, r)


def test_split_rows_and_workspace_bytes():
    L = qm.lib()
    assert [qm.split_rows(r) for r in (0, 1, 16, 17, 255)] == [0, 16, 16, 32, 256]
    assert L.qmoe_split_rows(-3) == -1
    w = qm._Weights(qm.INT4, 256, 2048, 512, 64, 0, 16, 0, 16, 0, 0, 0, 0, 0)
    assert L.qmoe_workspace_bytes(0, ctypes.byref(w), 2048, 8, 80) == qm.plan_bytes(2048, 8, 256, 80)
    assert L.qmoe_workspace_bytes(1, ctypes.byref(w), 2048, 8, 80) == 2048 * 2048 * 4
    assert L.qmoe_workspace_bytes(7, ctypes.byref(w), 2048, 8, 80) == 0
    assert L.qmoe_workspace_bytes(0, None, 2048, 8, 80) == 0


def test_boundary_accepts_any_n_and_long_k():
    """The argument checks pass (the call then stops at the device check: -7
    without a GPU) for any output row count n and any decode K that is a
    multiple of 32 up to 8192; FP8 keeps its 128-row scale blocks."""
    L = qm.lib()
    if L.qmoe_check_device() == 0:
        pytest.skip("a GPU is present: the calls would launch")
    P = ctypes.c_void_p(16)
    for n in (1, 40, 200, 1000):
        w = qm._Weights(qm.Q8_0, 1, n, 256, 0, 0, 16, 0, 16, 0, 0, 0, 0, 0)
        assert L.qmoe_qmm_dense(ctypes.byref(w), P, 1, 4, 0, P, 1, None) == -7
        w = qm._Weights(qm.INT4, 3, n, 256, 64, 0, 16, 0, 16, 0, 0, 0, 0, 0)
        assert L.qmoe_moe_gather_qmm(ctypes.byref(w), P, 4, 2, 80, P, 2, 0, None, 0, P, 2, None) == -7
    for k in (1408, 3072, 7168, 8192):
        w = qm._Weights(qm.Q8_0, 8, 24, k, 0, 0, 16, 0, 16, 0, 0, 0, 0, 0)
        assert L.qmoe_moe_gemv(ctypes.byref(w), P, 1, 2, P, P, 4, 2, P, 1, None) == -7
    w = qm._Weights(qm.Q8_0, 8, 24, 8256, 0, 0, 16, 0, 16, 0, 0, 0, 0, 0)
    assert L.qmoe_moe_gemv(ctypes.byref(w), P, 1, 2, P, P, 4, 2, P, 1, None) == -4
    w = qm._Weights(qm.MXFP4, 8, 24, 96, 0, 0, 16, 0, 16, 0, 0, 0, 0, 0)
    assert L.qmoe_moe_gemv(ctypes.byref(w), P, 1, 2, P, P, 4, 1, P, 1, None) == -3  # k % 64
    w = qm._Weights(qm.FP8, 1, 200, 256, 0, 0, 16, 0, 16, 0, 0, 0, 0, 0)
    assert L.qmoe_qmm_dense(ctypes.byref(w), P, 1, 4, 0, P, 1, None) == -3


def test_binding_rejects_mis_shaped_tensors():
    """The binding checks every caller-supplied tensor (shape, dtype,
    contiguity) before a pointer reaches the library."""
    torch = pytest.importorskip("torch")
    w = qm.DeviceWeights("int4", 4, 64, 128, 64, {})
    with pytest.raises(ValueError):                           # K mismatch
        qm.qmm_dense(w, torch.zeros((8, 96), dtype=torch.bfloat16))
    with pytest.raises(ValueError):                           # activations must be f16 / bf16
        qm.qmm_dense(w, torch.zeros((8, 128), dtype=torch.float32))
    with pytest.raises(ValueError):                           # not contiguous
        qm.qmm_dense(w, torch.zeros((128, 8), dtype=torch.bfloat16).t())
    with pytest.raises(ValueError):                           # ids must be int32
        qm.moe_plan(torch.zeros((4, 2), dtype=torch.int64), 4)
    ids = torch.zeros((4, 2), dtype=torch.int32)
    with pytest.raises(ValueError):                           # plan buffer too small
        qm.moe_plan(ids, 4, plan=torch.zeros(8, dtype=torch.int32))
    with pytest.raises(ValueError):                           # GATHER_TOKENS needs [T, K]
        qm.moe_gather_qmm(w, torch.zeros(4096, dtype=torch.int32), 4, 2, torch.zeros((5, 128), dtype=torch.bfloat16))
    wd = qm.DeviceWeights("int4", 4, 128, 128, 64, {})
    with pytest.raises(ValueError):                           # combine GEMV takes [B, topk, K]
        qm.moe_gemv(wd, torch.zeros((4, 2, 64), dtype=torch.bfloat16), ids, torch.zeros((4, 2)),
                    epilogue=qm.EPI_WEIGHTED_COMBINE)
    with pytest.raises(ValueError):                           # topk_w shape
        qm.moe_combine(torch.zeros((8, 64), dtype=torch.bfloat16), torch.zeros(4096, dtype=torch.int32), 4, 2, 4,
                       torch.zeros((4, 3)))
    with pytest.raises(ValueError):                           # out shape
        qm.combine_cast(torch.zeros((4, 64)), out=torch.zeros((4, 32), dtype=torch.bfloat16))

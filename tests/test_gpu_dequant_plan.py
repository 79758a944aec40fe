"""GPU parity: standalone dequantisation (bit-exact) and the routing plan
(exact integers) against the CPU oracle, through the C ABI."""
import struct

import numpy as np
import pytest

import block_quantized_moe_amd as qm
import oracle
import synth
from _helpers import upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bits_equal(gpu, ref, dtype):
    """Bit-exact comparison; NaNs only need to be NaN on both sides."""
    if dtype == "f32":
        g = gpu.detach().cpu().numpy().astype(np.float32)
        r = np.asarray(ref, np.float32)
        nan = np.isnan(r)
        assert np.array_equal(np.isnan(g), nan)
        assert np.array_equal(g[~nan].view(np.uint32), r[~nan].view(np.uint32))
    else:
        g = gpu.detach().cpu().view(torch.int16).numpy().view(np.uint16)
        r = np.asarray(ref, np.uint16)
        if dtype == "f16":
            gn = np.isnan(g.view(np.float16)); rn = np.isnan(r.view(np.float16))
        else:
            gn = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0); rn = ((r & 0x7F80) == 0x7F80) & ((r & 0x7F) != 0)
        assert np.array_equal(gn, rn)
        bad = np.nonzero(g[~rn] != r[~rn])[0]
        assert bad.size == 0, f"{bad.size} mismatches, first {g[~rn][bad[:4]]} vs {r[~rn][bad[:4]]}"


def _weights(fmt, rng):
    if fmt in ("q2_k", "iq2_xxs", "q4_k", "q6_k"):
        W = synth.weights(fmt, rng, 2, 40, 512)   # E*N a multiple of 16 (tiled layout)
    elif fmt == "int4":
        W = synth.int4(rng, 2, 40, 512, 64)   # E*N a multiple of 16 (tiled int4 layout)
    elif fmt == "mxfp4":
        W = synth.mxfp4(rng, 2, 40, 512)
    elif fmt == "fp8":
        W = synth.fp8(rng, 2, 128, 512)   # N and K multiples of the 128 x 128 scale block
    else:
        W = synth.q8_0(rng, 2, 40, 512)
    return W


def _plant_specials(W):
    """Edge scales and codes: NaN, inf, subnormal, signed zero, byte 0x80."""
    h = lambda b: np.frombuffer(struct.pack("<H", b), np.uint8)
    if W.fmt == "q8_0":
        for i, b in enumerate([0x7E00, 0x7C00, 0x0001, 0x8000, 0x03FF]):
            W.blocks[0, i, 0, 0:2] = h(b)
        W.blocks[0, 5, 1, 2:34] = 0x80
    elif W.fmt == "q2_k":
        W.blocks[0, 0, 0, 80:82] = h(0x7E00)
        W.blocks[0, 1, 0, 82:84] = h(0x0001)
        W.blocks[0, 2, 0, 80:82] = h(0x0003)
        W.blocks[0, 3, 0, 80:84] = 0
    elif W.fmt == "mxfp4":
        for i, e in enumerate([255, 0, 254, 1, 253, 127]):  # NaN, 2^-127, past fp32 for |v| >= 2, ...
            W.blocks[0, i, 0, 0] = e
        W.blocks[0, 7, 2, 1:] = 0x88   # -0 codes
    elif W.fmt == "fp8":
        f = np.float32
        for j, v in enumerate([f(np.nan), f(np.inf), f(1e-45), f(-0.0)]):
            W.scale[0, 0, j] = v
        W.scale[1, 0, 0] = f(3e38)                            # 3e38 * 448 overflows fp32
        W.qs[0, 0, 0:4] = [0x7F, 0xFF, 0x80, 0x01]          # NaN, NaN, -0, smallest subnormal
        W.qs[0, 1, 128:136] = [0x00, 0x07, 0x08, 0x7E, 0xFE, 0x87, 0x88, 0xF7]
    elif W.fmt == "q4_k":
        W.blocks[0, 0, 0, 0:2] = h(0x7E00)    # NaN d
        W.blocks[0, 1, 0, 2:4] = h(0x0001)    # subnormal dmin
        W.blocks[0, 2, 0, 0:2] = h(0x0003)    # subnormal d
        W.blocks[0, 3, 0, 0:4] = 0            # zero d and dmin
        W.blocks[0, 4, 1, 0:2] = h(0x7C00)    # inf d
    elif W.fmt == "q6_k":
        W.blocks[0, 0, 0, 208:210] = h(0x7E00)
        W.blocks[0, 1, 0, 208:210] = h(0x0001)
        W.blocks[0, 2, 0, 208:210] = h(0x8000)  # -0: values +-0
        W.blocks[0, 3, 1, 192:208] = 0x80       # scales -128
    elif W.fmt == "iq2_xxs":
        W.blocks[0, 0, 0, 0:2] = h(0x7E00)
        W.blocks[0, 1, 0, 0:2] = h(0x0001)
        W.blocks[0, 2, 0, 0:2] = h(0x8000)
    else:
        W.scale[0, 0, 0] = 0x7E00
        W.bias[0, 1, 0] = 0x7C00
        W.scale[0, 2, 0] = 0x0001
        W.bias[0, 2, 0] = 0x8001
    return W


@pytest.mark.parametrize("fmt", ["q8_0", "q2_k", "iq2_xxs", "int4", "mxfp4", "fp8", "q4_k", "q6_k"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dequant_bit_exact(fmt, dtype):
    W = _plant_specials(_weights(fmt, np.random.default_rng(17)))
    dw = upload(W)
    code = {"f32": qm.F32, "f16": qm.F16, "bf16": qm.BF16}[dtype]
    with np.errstate(invalid="ignore", over="ignore"):  # planted NaN / inf / out-of-range scales
        ref32 = oracle.dequant(W)
        ref = oracle.round_out(ref32, dtype) if dtype != "f32" else ref32
    out = qm.dequant(dw, code)
    torch.cuda.synchronize()
    _bits_equal(out.reshape(-1), ref.reshape(-1), dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dequant_mxfp4_every_code_and_exponent(dtype):
    # all 256 exponent bytes x all 16 codes, each exponent in its own block
    W = synth.mxfp4(np.random.default_rng(6), 1, 256, 64)
    W.blocks[0, :, :, 0] = np.arange(256, dtype=np.uint8)[:, None]
    codes = np.arange(32) % 16
    W.blocks[0, :, :, 1:] = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    code = {"f32": qm.F32, "f16": qm.F16, "bf16": qm.BF16}[dtype]
    out = qm.dequant(upload(W), code)
    torch.cuda.synchronize()
    ref32 = oracle.dequant(W)
    with np.errstate(over="ignore"):
        ref = oracle.round_out(ref32, dtype) if dtype != "f32" else ref32
    _bits_equal(out.reshape(-1), ref.reshape(-1), dtype)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_dequant_fp8_every_code(dtype):
    # all 256 E4M3 bytes in every row, under scales of 1, powers of two and random values
    rng = np.random.default_rng(8)
    W = synth.fp8(rng, 1, 256, 512)
    W.qs[0] = (np.arange(512)[None, :] + 37 * np.arange(256)[:, None]) % 256
    W.scale[0, 0, 0] = 1.0
    W.scale[0, 0, 1] = 2.0 ** -20
    W.scale[0, 1, 2] = 2.0 ** 10
    code = {"f32": qm.F32, "f16": qm.F16, "bf16": qm.BF16}[dtype]
    out = qm.dequant(upload(W), code)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        ref32 = oracle.dequant(W)
        ref = oracle.round_out(ref32, dtype) if dtype != "f32" else ref32
    _bits_equal(out.reshape(-1), ref.reshape(-1), dtype)


def test_dequant_iq2_xxs_every_index_and_sign():
    # every grid index x every sign field x every scale nibble appears
    rng = np.random.default_rng(5)
    W = synth.iq2_xxs(rng, 1, 64, 2048)
    grp = W.blocks[..., 2:66].reshape(-1, 8, 8)
    flat = np.arange(grp.shape[0] * 8)
    grp[:, :, 0:4] = (flat.reshape(-1, 8, 1) * 4 + np.arange(4)) % 256
    aux = ((flat % 128) | ((flat * 7 % 128) << 7) | ((flat * 3 % 128) << 14) | ((flat * 5 % 128) << 21)
           | ((flat % 16) << 28)).astype("<u4")
    grp[:, :, 4:8] = aux.reshape(-1, 8, 1).view(np.uint8).reshape(-1, 8, 4)
    W.blocks[..., 2:66] = grp.reshape(W.blocks[..., 2:66].shape)
    out = qm.dequant(upload(W), qm.F32)
    torch.cuda.synchronize()
    _bits_equal(out.reshape(-1), oracle.dequant(W).reshape(-1), "f32")


def _plan_case(T, k, E, bm, seed, bad=True, skew=False):
    rng = np.random.default_rng(seed)
    if skew:
        ids, _ = synth.routing_zipf(rng, T, E, k, 1.1)
    else:
        ids, _ = synth.routing_softmax(rng, T, E, k)
    if bad and T > 3:
        ids[1, 0] = -1
        ids[3, k - 1] = E + 5
    return ids


@pytest.mark.parametrize("T,k,E,bm,skew", [(300, 8, 64, 80, False), (1, 1, 4, 16, False),
                                           (2048, 8, 256, 64, False), (4096, 8, 256, 48, True),
                                           (513, 6, 1024, 32, False),
                                           # 64 and 66 chunks of 1024 pairs, Zipf-skewed
                                           (8192, 8, 256, 80, True), (8448, 8, 256, 80, True)])
def test_plan_exact(T, k, E, bm, skew):
    ids = _plan_case(T, k, E, bm, 7 + T, skew=skew)
    ref = oracle.plan(ids, E, bm)
    ids_d = torch.from_numpy(ids).cuda()
    plan = qm.moe_plan(ids_d, E, bm)
    torch.cuda.synchronize()
    v = {key: val.cpu().numpy() for key, val in qm.plan_views(plan, T, k, E).items()}
    h = v["header"]
    nt = len(ref["tiles"])
    assert h[0] == ref["dropped"] and h[1] == nt and h[2] == len(ref["sorted"]) and h[3] == bm
    assert np.array_equal(v["counts"], ref["counts"])
    assert np.array_equal(v["offsets"], ref["offsets"])
    assert np.array_equal(v["sorted"][:len(ref["sorted"])], ref["sorted"])
    # the tile set is unique; its order is the kernel's schedule: full tiles
    # first (expert order), then the partial ones (expert order)
    got = v["tiles"][:nt, :3]
    key = lambda t: np.lexsort((t[:, 1], t[:, 0]))
    assert np.array_equal(got[key(got)], ref["tiles"][key(ref["tiles"])])
    full = got[:, 2] == bm
    assert not np.any(full[np.argmin(full):]) if not full.all() else True
    for part in (got[full], got[~full]):
        assert np.all(np.diff(part[:, 0] * (T * k + 1) + part[:, 1]) > 0)
    inv = np.full(T * k, -1)
    inv[ref["sorted"]] = np.arange(len(ref["sorted"]))
    assert np.array_equal(v["inv"], inv)

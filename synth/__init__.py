"""Seeded synthetic inputs for the block-quantized MoE expert matmul.

This module only *draws* inputs: random quant codes, fp16 scales, activations
and routing decisions, packed into the on-disk block layouts below.  It holds
none of the method's arithmetic (no dequantisation, no matmul, no combine), so
both the CPU oracle and the HIP path can consume its output without sharing
any code with each other.

On-disk layouts produced here (one block per row-chunk of K, little endian):

* Q8_0      34 B / 32 values : [fp16 d][32 x int8 q]
* Q2_K      84 B / 256 values: [16 B scale|min nibbles][64 B 2-bit codes][fp16 d][fp16 dmin]
* IQ2_XXS   66 B / 256 values: [fp16 d] then 8 groups of [4 grid-index bytes][u32 aux]
* Q4_K     144 B / 256 values: [fp16 d][fp16 dmin][12 B packed 6-bit scales/mins][128 B 4-bit codes]
* Q6_K     210 B / 256 values: [128 B low nibbles][64 B high bit pairs][16 x int8 scale][fp16 d]
* int4      MLX-style, already split: qs u32 [E, N, K/8] (8 nibbles per word),
            scale / bias fp16 [E, N, K/group]

Weight tensors are W[E, N, K] with the blocks running along K (the reduction
dimension), so y = x . W^T.

Distributions follow the workload descriptions (activations N(0,1); Q8_0 codes
uniform in [-127, 127] with an fp16 scale |N(0,0.02)|/127; int4 codes uniform
0..15 with group-64 fp16 scale and bias; IQ2_XXS grid of small positive
magnitudes {8, 25, 43}).  Scale distributions the workload text leaves open
are chosen so every format yields weights of roughly 0.02 magnitude.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Byte sizes of the on-disk blocks.
Q8_0_BLOCK = 32
Q8_0_BYTES = 34
QK_K = 256
Q2_K_BYTES = 84
IQ2_XXS_BYTES = 66
Q4_K_BYTES = 144
Q6_K_BYTES = 210
INT4_GROUP = 64
MXFP4_BLOCK = 32
MXFP4_BYTES = 17

# Child-stream order for one configuration's SeedSequence.
STREAMS = ("activations", "router", "w_gate_up", "w_down", "shared")
GRID_SEED = 22
GRID_MAGNITUDES = (8, 25, 43)


def streams(config_id: int) -> dict[str, np.random.Generator]:
    """Independent generators for one configuration, spawned in a fixed order."""
    kids = np.random.SeedSequence(config_id).spawn(len(STREAMS))
    return {name: np.random.default_rng(k) for name, k in zip(STREAMS, kids)}


# ---------------------------------------------------------------------------
# storage-format helpers for *drawing* inputs (fp16 / bf16 bit patterns)
# ---------------------------------------------------------------------------

def f16_bits(a) -> np.ndarray:
    """IEEE binary16 bit patterns (round to nearest even) of float values."""
    return np.asarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def bf16_bits(a) -> np.ndarray:
    """bfloat16 bit patterns of float values, round to nearest even.

    Used only to draw bf16 activations; inputs here are finite.
    """
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


# ---------------------------------------------------------------------------
# weight containers
# ---------------------------------------------------------------------------

@dataclass
class QWeights:
    """A stacked expert weight tensor W[E, N, K] in its on-disk form.

    fmt: "q8_0" | "q2_k" | "iq2_xxs" | "mxfp4" | "int4" | "fp8" | "q4_k" | "q6_k".
    blocks: uint8 [E, N, K/block, block_bytes] for the GGUF-style formats.
    qs/scale/bias: int4 arrays (uint32 [E,N,K/8], uint16 fp16 bits [E,N,K/group]);
    for fp8, qs uint8 E4M3 bytes [E,N,K] and scale fp32 [E,N/128,K/128].
    grid: uint8 [256, 8] magnitude table (IQ2_XXS only).
    """
    fmt: str
    E: int
    N: int
    K: int
    group: int = 0
    blocks: np.ndarray | None = None
    qs: np.ndarray | None = None
    scale: np.ndarray | None = None
    bias: np.ndarray | None = None
    grid: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    def expert_rows(self, e: int, rows) -> "QWeights":
        """A view restricted to expert e and the given output rows (E=1)."""
        rows = np.asarray(rows)
        if self.fmt == "fp8":
            # group = weight rows per scale row: 1 here (one scale row per selected row)
            return QWeights("fp8", 1, len(rows), self.K, 1, qs=self.qs[e, rows][None],
                            scale=self.scale[e, rows // 128][None])
        if self.fmt == "int4":
            return QWeights("int4", 1, len(rows), self.K, self.group,
                            qs=self.qs[e, rows][None], scale=self.scale[e, rows][None],
                            bias=self.bias[e, rows][None])
        return QWeights(self.fmt, 1, len(rows), self.K, self.group,
                        blocks=self.blocks[e, rows][None], grid=self.grid)

    @property
    def nbytes(self) -> int:
        if self.fmt == "fp8":
            return int(self.qs.nbytes + self.scale.nbytes)
        if self.fmt == "int4":
            return int(self.qs.nbytes + self.scale.nbytes + self.bias.nbytes)
        return int(self.blocks.nbytes)


def iq2_grid(seed: int = GRID_SEED) -> np.ndarray:
    """Seeded stand-in for the IQ2_XXS magnitude grid: 256 rows x 8 bytes."""
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    return rng.choice(np.array(GRID_MAGNITUDES, dtype=np.uint8), size=(256, 8))


def _absn(rng, shape, sigma):
    return np.abs(rng.standard_normal(shape, dtype=np.float32)) * np.float32(sigma)


def q8_0(rng: np.random.Generator, E: int, N: int, K: int) -> QWeights:
    assert K % Q8_0_BLOCK == 0
    nb = K // Q8_0_BLOCK
    blocks = np.empty((E, N, nb, Q8_0_BYTES), dtype=np.uint8)
    d = f16_bits(_absn(rng, (E, N, nb), 0.02) / np.float32(127.0))
    blocks[..., 0:2] = d[..., None].view(np.uint8).reshape(E, N, nb, 2)
    q = rng.integers(-127, 128, size=(E, N, nb, 32), dtype=np.int16).astype(np.int8)
    blocks[..., 2:34] = q.view(np.uint8)
    return QWeights("q8_0", E, N, K, Q8_0_BLOCK, blocks=blocks)


def q2_k(rng: np.random.Generator, E: int, N: int, K: int) -> QWeights:
    assert K % QK_K == 0
    nb = K // QK_K
    blocks = np.empty((E, N, nb, Q2_K_BYTES), dtype=np.uint8)
    blocks[..., 0:80] = rng.integers(0, 256, size=(E, N, nb, 80), dtype=np.uint8)
    d = f16_bits(_absn(rng, (E, N, nb), 0.02) / np.float32(12.0))
    dmin = f16_bits(_absn(rng, (E, N, nb), 0.02) / np.float32(8.0))
    blocks[..., 80:82] = d[..., None].view(np.uint8).reshape(E, N, nb, 2)
    blocks[..., 82:84] = dmin[..., None].view(np.uint8).reshape(E, N, nb, 2)
    return QWeights("q2_k", E, N, K, QK_K, blocks=blocks)


def q4_k(rng: np.random.Generator, E: int, N: int, K: int) -> QWeights:
    assert K % QK_K == 0
    nb = K // QK_K
    blocks = np.empty((E, N, nb, Q4_K_BYTES), dtype=np.uint8)
    d = f16_bits(_absn(rng, (E, N, nb), 0.02) / np.float32(240.0))
    dmin = f16_bits(_absn(rng, (E, N, nb), 0.02) / np.float32(32.0))
    blocks[..., 0:2] = d[..., None].view(np.uint8).reshape(E, N, nb, 2)
    blocks[..., 2:4] = dmin[..., None].view(np.uint8).reshape(E, N, nb, 2)
    blocks[..., 4:144] = rng.integers(0, 256, size=(E, N, nb, 140), dtype=np.uint8)
    return QWeights("q4_k", E, N, K, QK_K, blocks=blocks)


def q6_k(rng: np.random.Generator, E: int, N: int, K: int) -> QWeights:
    assert K % QK_K == 0
    nb = K // QK_K
    blocks = np.empty((E, N, nb, Q6_K_BYTES), dtype=np.uint8)
    blocks[..., 0:192] = rng.integers(0, 256, size=(E, N, nb, 192), dtype=np.uint8)
    blocks[..., 192:208] = rng.integers(-64, 64, size=(E, N, nb, 16), dtype=np.int16).astype(np.int8).view(np.uint8)
    d = f16_bits(_absn(rng, (E, N, nb), 0.02) / np.float32(512.0))
    blocks[..., 208:210] = d[..., None].view(np.uint8).reshape(E, N, nb, 2)
    return QWeights("q6_k", E, N, K, QK_K, blocks=blocks)


def iq2_xxs(rng: np.random.Generator, E: int, N: int, K: int,
            grid: np.ndarray | None = None) -> QWeights:
    assert K % QK_K == 0
    nb = K // QK_K
    blocks = np.empty((E, N, nb, IQ2_XXS_BYTES), dtype=np.uint8)
    d = f16_bits(_absn(rng, (E, N, nb), 0.02) / np.float32(50.0))
    blocks[..., 0:2] = d[..., None].view(np.uint8).reshape(E, N, nb, 2)
    idx = rng.integers(0, 256, size=(E, N, nb, 8, 4), dtype=np.uint8)
    sgn = rng.integers(0, 128, size=(E, N, nb, 8, 4), dtype=np.uint32)
    scl = rng.integers(0, 16, size=(E, N, nb, 8), dtype=np.uint32)
    aux = (sgn[..., 0] | (sgn[..., 1] << 7) | (sgn[..., 2] << 14) | (sgn[..., 3] << 21)
           | (scl << 28)).astype("<u4")
    grp = np.empty((E, N, nb, 8, 8), dtype=np.uint8)
    grp[..., 0:4] = idx
    grp[..., 4:8] = aux[..., None].view(np.uint8).reshape(E, N, nb, 8, 4)
    blocks[..., 2:66] = grp.reshape(E, N, nb, 64)
    return QWeights("iq2_xxs", E, N, K, QK_K, blocks=blocks,
                    grid=iq2_grid() if grid is None else grid)


def int4(rng: np.random.Generator, E: int, N: int, K: int, group: int = INT4_GROUP) -> QWeights:
    assert K % group == 0 and group % 8 == 0
    qs = rng.integers(0, 2**32, size=(E, N, K // 8), dtype=np.uint64).astype(np.uint32)
    s32 = _absn(rng, (E, N, K // group), 0.02) / np.float32(7.5)
    s = f16_bits(s32)
    s_back = s.view(np.float16).astype(np.float32)
    b = f16_bits(-7.5 * s_back + 0.5 * s_back * rng.standard_normal(s_back.shape, dtype=np.float32))
    return QWeights("int4", E, N, K, group, qs=qs, scale=s, bias=b)


def mxfp4(rng: np.random.Generator, E: int, N: int, K: int) -> QWeights:
    """MXFP4 blocks: the E8M0 exponent byte (2^-9 .. 2^-5 scales, so the
    largest code, 6, gives weights up to about 0.19) and 16 bytes of uniform
    random 4-bit codes."""
    assert K % MXFP4_BLOCK == 0
    nb = K // MXFP4_BLOCK
    blocks = np.empty((E, N, nb, MXFP4_BYTES), dtype=np.uint8)
    blocks[..., 0] = rng.integers(118, 123, size=(E, N, nb), dtype=np.uint8)
    blocks[..., 1:] = rng.integers(0, 256, size=(E, N, nb, 16), dtype=np.uint8)
    return QWeights("mxfp4", E, N, K, MXFP4_BLOCK, blocks=blocks)


def fp8(rng: np.random.Generator, E: int, N: int, K: int) -> QWeights:
    """FP8 E4M3 block weights: bytes with exponent fields 4..10 (magnitudes
    1/8 .. 15; field 4 + (r mod 7) of a uniform byte r, so nearly uniform) and
    uniform signs and mantissas (no NaN codes), and fp32 scales |N(0, 0.02)| / 8
    per 128 x 128 block.  Drawn one expert at a time (two uniform bytes per
    weight) so full-size expert stacks stay quick to generate."""
    assert N % 128 == 0 and K % 128 == 0
    qs = np.empty((E, N, K), np.uint8)
    ex = ((4 + np.arange(256) % 7) << 3).astype(np.uint8)       # exponent field of byte r
    for e in range(E):
        r = np.frombuffer(rng.bytes(2 * N * K), np.uint8).reshape(2, N, K)
        qs[e] = (r[0] & np.uint8(0x87)) | ex[r[1]]                 # sign and mantissa | exponent
    scale = (_absn(rng, (E, N // 128, K // 128), 0.02) / np.float32(8.0)).astype(np.float32)
    return QWeights("fp8", E, N, K, 128, qs=qs, scale=scale)  # group: weight rows per scale row


def weights(fmt: str, rng, E, N, K, **kw) -> QWeights:
    return {"q8_0": q8_0, "q2_k": q2_k, "iq2_xxs": iq2_xxs, "mxfp4": mxfp4, "int4": int4,
            "fp8": fp8, "q4_k": q4_k, "q6_k": q6_k}[fmt](rng, E, N, K, **kw)


# ---------------------------------------------------------------------------
# activations and routing
# ---------------------------------------------------------------------------

def activations(rng: np.random.Generator, T: int, K: int, dtype: str) -> np.ndarray:
    """N(0,1) activations as uint16 bit patterns of fp16 or bf16."""
    x = rng.standard_normal((T, K), dtype=np.float32)
    return f16_bits(x) if dtype == "f16" else bf16_bits(x)


def _pairs_from_keys(keys: np.ndarray, k: int):
    """k distinct experts per row, the k largest keys (continuous keys, so no
    ties in practice), and the pair weights the workload text names: a
    softmax over the k selected keys, exp(l_j - l_0) / sum_i exp(l_i - l_0)
    in fp64 (l_0 the largest), stored as fp32.  An input recipe drawn on the
    host, not the device router."""
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(keys.astype(np.float64), ids, axis=1)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


def routing_softmax(rng: np.random.Generator, T: int, E: int, k: int):
    """Uniform routing of the Qwen-shaped workloads: N(0,1) router logits per
    token and expert, the top k of each row, weights the softmax over the
    selected logits."""
    return _pairs_from_keys(rng.standard_normal((T, E), dtype=np.float32), k)


def routing_zipf(rng: np.random.Generator, T: int, E: int, k: int, alpha: float = 1.1):
    """Skewed routing: expert popularity p ~ rank^-alpha over a seeded
    permutation; keys log p + Gumbel(0,1) act as the router logits, so the
    top k of a row samples experts without replacement in proportion to p;
    weights the softmax over the selected keys."""
    perm = rng.permutation(E)
    p = np.empty(E)
    p[perm] = np.arange(1, E + 1, dtype=np.float64) ** (-alpha)
    p /= p.sum()
    keys = (np.log(p)[None, :] + rng.gumbel(size=(T, E))).astype(np.float32)
    return _pairs_from_keys(keys, k)


def router_logits(rng: np.random.Generator, T: int, E: int, dtype: str, sigma: float = 1.0) -> np.ndarray:
    """Router logits N(0, sigma^2) [T, E]: float32, or uint16 bit patterns of
    fp16 / bf16."""
    x = (sigma * rng.standard_normal((T, E))).astype(np.float32)
    if dtype == "f32":
        return x
    return f16_bits(x) if dtype == "f16" else bf16_bits(x)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

@dataclass
class MoEInputs:
    name: str
    act: str              # "f16" | "bf16"
    out: str              # combine output dtype
    T: int
    H: int
    I: int
    E: int
    k: int
    x: np.ndarray         # uint16 [T, H]
    ids: np.ndarray       # int32 [T, k]
    w: np.ndarray         # float32 [T, k]
    w_gate_up: QWeights   # [E, 2I, H]: rows 0..I-1 gate, I..2I-1 up
    w_down: QWeights      # [E, H, I]
    shared_gate_up: QWeights | None = None   # [1, 2Is, H]
    shared_down: QWeights | None = None      # [1, H, Is]
    projections: list = field(default_factory=list)  # dense [1, H, H] each


def dense_q8_0(config_id: int = 0, M: int = 32, N: int = 256, K: int = 2048):
    """Dense Q8_0 qmm: fp16 activations [M, K], weights [1, N, K]."""
    s = streams(config_id)
    x = activations(s["activations"], M, K, "f16")
    w = q8_0(s["w_gate_up"], 1, N, K)
    return x, w


def moe(config_id: int, *, T: int, H: int, I: int, E: int, k: int,
        gate_up_fmt: str, down_fmt: str, act: str, out: str,
        routing: str = "softmax", shared_I: int = 0, n_proj: int = 0,
        name: str = "") -> MoEInputs:
    s = streams(config_id)
    x = activations(s["activations"], T, H, act)
    if routing == "zipf":
        ids, w = routing_zipf(s["router"], T, E, k)
    else:
        ids, w = routing_softmax(s["router"], T, E, k)
    wgu = weights(gate_up_fmt, s["w_gate_up"], E, 2 * I, H)
    wd = weights(down_fmt, s["w_down"], E, H, I)
    inp = MoEInputs(name, act, out, T, H, I, E, k, x, ids, w, wgu, wd)
    if shared_I:
        inp.shared_gate_up = q8_0(s["shared"], 1, 2 * shared_I, H)
        inp.shared_down = q8_0(s["shared"], 1, H, shared_I)
    for _ in range(n_proj):
        inp.projections.append(q8_0(s["shared"], 1, H, H))
    return inp


# Full-size workload shapes (sizes as the workload descriptions give them).
QWEN_A3B = dict(H=2048, I=512, E=256, k=8, gate_up_fmt="int4", down_fmt="int4",
                act="bf16", out="bf16")
DSV4_FLASH = dict(H=4096, I=2048, E=256, k=6, gate_up_fmt="iq2_xxs", down_fmt="q2_k",
                  act="f16", out="f16")
MIXED_FFN = dict(H=4096, I=2048, E=256, k=8, gate_up_fmt="iq2_xxs", down_fmt="q2_k",
                 act="f16", out="bf16", routing="zipf", shared_I=2048, n_proj=4)


def qwen_a3b_prefill(T: int = 2048, **over) -> MoEInputs:
    return moe(1, T=T, name="qwen3.6-a3b-int4-prefill", **{**QWEN_A3B, **over})


def qwen_a3b_decode(B: int, **over) -> MoEInputs:
    return moe(2, T=B, name=f"qwen3.6-a3b-int4-decode-b{B}", **{**QWEN_A3B, **over})


def dsv4_flash_prefill(T: int = 2048, **over) -> MoEInputs:
    return moe(3, T=T, name="dsv4-flash-iq2xxs-q2k-prefill", **{**DSV4_FLASH, **over})


def dsv4_flash_mxfp4_prefill(T: int = 2048, **over) -> MoEInputs:
    """The DSv4-Flash expert shapes with its native MXFP4 expert weights."""
    fmt = dict(gate_up_fmt="mxfp4", down_fmt="mxfp4")
    return moe(5, T=T, name="dsv4-flash-mxfp4-prefill", **{**DSV4_FLASH, **fmt, **over})


def dsv4_flash_fp8_prefill(T: int = 2048, **over) -> MoEInputs:
    """The DSv4-Flash expert shapes with FP8 E4M3 block expert weights (the
    DeepSeek V3 storage that V4 inherits: fp32 scale per 128 x 128 block)."""
    fmt = dict(gate_up_fmt="fp8", down_fmt="fp8")
    return moe(6, T=T, name="dsv4-flash-fp8-prefill", **{**DSV4_FLASH, **fmt, **over})


def dsv4_flash_kquant_prefill(T: int = 2048, **over) -> MoEInputs:
    """The DSv4-Flash expert shapes with Q4_K gate/up and Q6_K down weights
    (the k-quant formats the pages name; layouts read as GGUF's)."""
    fmt = dict(gate_up_fmt="q4_k", down_fmt="q6_k")
    return moe(7, T=T, name="dsv4-flash-kquant-prefill", **{**DSV4_FLASH, **fmt, **over})


def mixed_ffn(T: int = 8192, **over) -> MoEInputs:
    return moe(4, T=T, name="mixed-format-moe-ffn", **{**MIXED_FFN, **over})

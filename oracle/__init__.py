"""CPU oracle for the block-quantized MoE expert matmul -- TEST INFRASTRUCTURE.

This package is the plain, slow, obviously-correct reference that the HIP path
is checked against.  Only the tests, the smoke entry point and the benchmark's
CPU-baseline leg may import it; the product path never calls it, and it shares
no code with the HIP library (it decodes the on-disk blocks itself, it does not
use the library's block splitter).

Precision: every weight is decoded to fp32 by the format's formula (exact for
every format, see each decoder), widened to fp64, and contracted in fp64.
Output roundings to fp16 / bf16 are round-to-nearest-even written out below.

Sources (web pages the method is described on):
  [GGUF]  "feat(gguf,dsv4): GGUF block-dequant + DSv4 kernel surface (WIP)",
          PR body sections "Design -- CPU-side decomposition" and "Kernels"
          items 1-3, and the follow-up commit that fixes IQ2_XXS sign
          reconstruction (two lookup tables).
  [DSV4]  "metal: DSV4 M1 Ultra prefill/decode campaign", PR body (tiled MoE
          prefill GEMM, q2_K SoA down twin, sum-folded q2_K down projection)
          and the review-fix commit (moe_mm_id AoS qs base at 84*blk+16).
  [BAGEL] "Everything Bagel 2", commits on the scalar-FMA top-K accumulator,
          the GPU MoE router top-K and the expert-indexed int4 GEMV
          ([nExperts, outDim, inDim/8] u32 weights with scales and biases),
          and the fused swiglu commit (silu(g) * u).
          Also the MXFP4 dequant commit (OCP MX v1.0 blocks) and the FP8
          block dequant commit (E4M3 bytes, fp32 scale per 128 x 128).
  [SHIM]  "WIP: metaltile shim -- Qwen3.6 mt_qmm_mma / mt_moe_gather dispatch
          from VLLMBridge", PR body (dense qmm smoke cell M=32 N=256 K=2048).

Readings where the pages are silent (each repeated at the function):
  * Q2_K: low nibble of a scale byte is the sub-block scale, high nibble its
    min; element e of a super-block sits in code byte 32*(e//128) + e%32 at bit
    2*((e%128)//32); d then dmin follow the 64 code bytes.
  * IQ2_XXS: the 4 scale bits are the top nibble of each group's aux word and
    the group scale is d * (0.5 + s) / 4; fp16 d leads the 66-byte block.
  * Sign table: entry i is i with bit 7 set iff i has an odd number of set
    bits (the "even-parity 8th sign").
  * int4: nibble i of word w is element 8*w + i (low nibble first).
  * MXFP4: "low nibble first" read as element 2i in the low nibble of code
    byte i (adjacent elements share a byte).
  * Q4_K and Q6_K: the pages only name these formats; the oracle reads them
    as the GGUF k-quant blocks (layouts at dequant_q4_k / dequant_q6_k).
    PARITY UNPINNED: nothing on the pages fixes these layouts, so the pins in
    tests/test_oracle_kquants.py check only the decoders' arithmetic and bit
    bookkeeping against that reading.
  * Routers: equal scores select the lower expert index first; the DSv4
    sqrtsoftplus gather weight is the unbiased score times the routed scaling
    factor, with no renormalisation (none is stated); the softmax-then-bias
    router selects on p + bias and weights the selected p renormalised.
Parity pins for every function live in tests/test_oracle_*.py.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f16_to_f64", "bf16_to_f64", "act_to_f64", "round_f16", "round_bf16",
    "iq2_signs", "dequant", "dequant_q8_0", "dequant_q2_k", "dequant_iq2_xxs",
    "q4_k_scales_mins", "dequant_q4_k", "dequant_q6_k",
    "e2m1_value", "e8m0_scale", "dequant_mxfp4", "e4m3_value", "dequant_fp8_block",
    "dequant_int4", "dequant_rows", "qmm", "silu", "plan", "moe_gate_up",
    "moe_down_combine", "moe_ffn", "moe_gate_up_rows", "moe_down_rows",
    "router_topk_softmax", "router_sqrtsoftplus", "gated_shared_residual", "combine_pairs",
    "router_softmax_bias_scores",
]

# ---------------------------------------------------------------------------
# scalar storage formats
# ---------------------------------------------------------------------------

def f16_to_f64(bits) -> np.ndarray:
    """fp16 bit patterns -> float64 (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact): bf16 is the top half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def act_to_f64(bits, dtype: str) -> np.ndarray:
    return f16_to_f64(bits) if dtype == "f16" else bf16_to_f64(bits)


def round_f16(v) -> np.ndarray:
    """fp32/fp64 -> fp16 bit patterns, IEEE round to nearest even, subnormals kept."""
    return np.asarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_bf16(v) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even; NaN stays NaN."""
    f = np.asarray(v, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    r[nan] = ((u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040))
    return r


def round_out(v, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return round_f16(v)
    if dtype == "bf16":
        return round_bf16(v)
    return np.asarray(v, dtype=np.float32)


def out_to_f64(a, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    return act_to_f64(a, dtype)


# ---------------------------------------------------------------------------
# block formats -> fp32  [GGUF "Kernels" 1-3]
# ---------------------------------------------------------------------------

def _f16_field(blocks: np.ndarray, off: int) -> np.ndarray:
    """fp16 little-endian field at byte offset `off` of every block, as fp32."""
    b = np.ascontiguousarray(blocks[..., off:off + 2])
    return b.view("<u2")[..., 0].view(np.float16).astype(np.float32)


def dequant_q8_0(blocks: np.ndarray) -> np.ndarray:
    """Q8_0 [GGUF "Kernels" 1]: 32 signed bytes share one scale;
    value = code * scale.  On disk the fp16 scale precedes the 32 codes.
    code * scale is exact in fp32 (8 x 11 significant bits).
    blocks: uint8 [..., 34] -> fp32 [..., 32]."""
    d = _f16_field(blocks, 0)
    q = np.ascontiguousarray(blocks[..., 2:34]).view(np.int8).astype(np.float32)
    return q * d[..., None]


def dequant_q2_k(blocks: np.ndarray) -> np.ndarray:
    """Q2_K [GGUF "Kernels" 2; DSV4 review fix: codes at byte 16 of 84]:
    a 256-value super-block of 16 sub-blocks of 16 values.  Sub-block s has a
    4-bit scale a_s (low nibble of byte s) and a 4-bit min m_s (high nibble);
    the super-block has fp16 d and dmin.  value = (d*a_s)*q - (dmin*m_s) with the
    2-bit code q of element e at code byte 32*(e//128) + e%32, bit 2*((e%128)//32).
    d*a*q and dmin*m are exact in fp32, so only the subtraction rounds.
    blocks: uint8 [..., 84] -> fp32 [..., 256]."""
    sc = blocks[..., 0:16]
    codes = blocks[..., 16:80]
    d = _f16_field(blocks, 80)
    dmin = _f16_field(blocks, 82)
    e = np.arange(256)
    byte = codes[..., 32 * (e // 128) + (e % 32)]
    q = ((byte >> (2 * ((e % 128) // 32)).astype(np.uint8)) & 3).astype(np.float32)
    sub = sc[..., e // 16]
    a = (sub & 15).astype(np.float32)
    m = (sub >> 4).astype(np.float32)
    dl = d[..., None] * a
    ml = dmin[..., None] * m
    return dl * q - ml


def q4_k_scales_mins(packed: np.ndarray):
    """The 8 six-bit (scale, min) pairs of a Q4_K super-block from its 12
    packed bytes (reading of the GGUF k-quant layout; parity unpinned).
    Sub-blocks 0-3: scale = low 6 bits of byte j, min = low 6 bits of byte
    j + 4.  Sub-blocks 4-7: the low 4 bits come from byte j + 4 (scale: its
    low nibble, min: its high nibble) and the top 2 bits from the spare top
    bits of bytes j - 4 (scale) and j (min).
    packed: uint8 [..., 12] -> (scale, min) uint8 [..., 8] each."""
    b = packed.astype(np.uint8)
    sc = np.empty(b.shape[:-1] + (8,), np.uint8)
    mn = np.empty(b.shape[:-1] + (8,), np.uint8)
    for j in range(4):
        sc[..., j] = b[..., j] & 63
        mn[..., j] = b[..., j + 4] & 63
        sc[..., j + 4] = (b[..., j + 8] & 15) | ((b[..., j] >> 6) << 4)
        mn[..., j + 4] = (b[..., j + 8] >> 4) | ((b[..., j + 4] >> 6) << 4)
    return sc, mn


def dequant_q4_k(blocks: np.ndarray) -> np.ndarray:
    """Q4_K (named by the pages; layout read as the GGUF k-quant block,
    parity unpinned): a 256-value super-block of 8 sub-blocks of 32 values,
    144 bytes = fp16 d, fp16 dmin, 12 bytes of packed six-bit scales and
    mins (q4_k_scales_mins), 128 code bytes.  Element e sits in code byte
    32*(e//64) + e%32, low nibble when e%64 < 32, else high nibble.
    value = (d*sc_j)*q - dmin*m_j for sub-block j = e//32; d*sc*q (11 + 6 + 4
    bits) and dmin*m are exact in fp32, so only the subtraction rounds.
    blocks: uint8 [..., 144] -> fp32 [..., 256]."""
    d = _f16_field(blocks, 0)
    dmin = _f16_field(blocks, 2)
    sc, mn = q4_k_scales_mins(blocks[..., 4:16])
    codes = blocks[..., 16:144]
    e = np.arange(256)
    byte = codes[..., 32 * (e // 64) + (e % 32)]
    q = np.where(e % 64 < 32, byte & 15, byte >> 4).astype(np.float32)
    j = e // 32
    return (d[..., None] * sc[..., j].astype(np.float32)) * q - dmin[..., None] * mn[..., j].astype(np.float32)


def dequant_q6_k(blocks: np.ndarray) -> np.ndarray:
    """Q6_K (named by the pages; layout read as the GGUF k-quant block,
    parity unpinned): a 256-value super-block of 16 sub-blocks of 16 values,
    210 bytes = 128 bytes of low nibbles, 64 bytes of high bit pairs, 16
    signed scale bytes, fp16 d.  Element e = 128*n + 32*p + l (n < 2, p < 4,
    l < 32): low 4 bits from byte 64*n + 32*(p % 2) + l of the first array
    (low nibble for p < 2, high for p >= 2), top 2 bits from byte 32*n + l of
    the second array at bits 2p, 2p+1; code q in 0..63.
    value = (d*sc_s)*(q - 32) for sub-block s = e//16; d*sc is exact in fp32,
    the product with q - 32 rounds once.
    blocks: uint8 [..., 210] -> fp32 [..., 256]."""
    ql = blocks[..., 0:128]
    qh = blocks[..., 128:192]
    sc = np.ascontiguousarray(blocks[..., 192:208]).view(np.int8).astype(np.float32)
    d = _f16_field(blocks, 208)
    e = np.arange(256)
    n, p, l = e // 128, (e % 128) // 32, e % 32
    lo = ql[..., 64 * n + 32 * (p % 2) + l]
    lo = np.where(p < 2, lo & 15, lo >> 4)
    hi = (qh[..., 32 * n + l] >> (2 * p).astype(np.uint8)) & 3
    q = (lo | (hi << 4)).astype(np.float32) - np.float32(32.0)
    return (d[..., None] * sc[..., e // 16]) * q


def iq2_signs() -> np.ndarray:
    """The 128-entry IQ2_XXS sign-mask table [GGUF IQ2_XXS sign-fix commit]:
    entry i keeps the 7 stored sign bits and adds an 8th sign bit so that the
    number of negated values in the octet is even.  uint8 [128]."""
    out = np.zeros(128, dtype=np.uint8)
    for i in range(128):
        ones = bin(i).count("1")
        out[i] = i | ((ones % 2) << 7)
    return out


def dequant_iq2_xxs(blocks: np.ndarray, grid: np.ndarray, signs: np.ndarray | None = None) -> np.ndarray:
    """IQ2_XXS [GGUF "Kernels" 3 and the sign-fix commit]: a 256-value
    super-block with fp16 d, then 8 groups of 32 values.  Each group stores 4
    grid-index bytes and a u32 aux word.  Octet j of the group takes its 8
    magnitudes from grid row idx_j; its sign mask is signs[(aux >> 7j) & 127]
    and bit l of the mask negates element l of the octet.  The group scale is
    d * (0.5 + (aux >> 28)) / 4 (reading: top nibble of aux holds the scale).
    d*(0.5+s)/4 * g is exact in fp32 (11 + 5 + 8 significant bits).
    blocks: uint8 [..., 66] -> fp32 [..., 256]."""
    if signs is None:
        signs = iq2_signs()
    d = _f16_field(blocks, 0)
    grp = np.ascontiguousarray(blocks[..., 2:66]).reshape(blocks.shape[:-1] + (8, 8))
    idx = grp[..., 0:4]                                     # [..., 8, 4]
    aux = np.ascontiguousarray(grp[..., 4:8]).view("<u4")[..., 0].astype(np.uint32)  # [..., 8]
    s = (aux >> 28).astype(np.float32)
    db = d[..., None] * (np.float32(0.5) + s) * np.float32(0.25)   # [..., 8]
    mag = grid[idx].astype(np.float32)                      # [..., 8, 4, 8]
    j = np.arange(4, dtype=np.uint32)
    field_ = (aux[..., None] >> (7 * j)) & 127              # [..., 8, 4]
    mask = signs[field_]                                    # [..., 8, 4]
    lbit = (mask[..., None] >> np.arange(8, dtype=np.uint8)) & 1   # [..., 8, 4, 8]
    sgn = np.where(lbit == 1, np.float32(-1.0), np.float32(1.0))
    w = db[..., None, None] * mag * sgn
    return w.reshape(blocks.shape[:-1] + (256,))


def dequant_int4(qs: np.ndarray, scale: np.ndarray, bias: np.ndarray, group: int) -> np.ndarray:
    """int4 affine [BAGEL expert-indexed int4 GEMV commit: stacked
    [nExperts, outDim, inDim/8] u32 weights plus per-group scales and biases]:
    value = s * q + b per group of `group` values along K; nibble i of word w
    is element 8w + i (reading: low nibble first).  s*q is exact in fp32, the
    +b rounds once.  qs uint32 [..., K/8]; scale/bias fp16 bits [..., K/group]
    -> fp32 [..., K]."""
    K = qs.shape[-1] * 8
    sh = (4 * np.arange(8, dtype=np.uint32))
    q = ((qs[..., :, None] >> sh) & 15).astype(np.float32).reshape(qs.shape[:-1] + (K,))
    s = np.asarray(scale, np.uint16).view(np.float16).astype(np.float32)
    b = np.asarray(bias, np.uint16).view(np.float16).astype(np.float32)
    s = np.repeat(s, group, axis=-1)
    b = np.repeat(b, group, axis=-1)
    return s * q + b


def e2m1_value(code) -> np.ndarray:
    """The FP4 E2M1 element of the OCP MX format [GGUF, the MXFP4 dequant
    commit, "Format"]: bit 3 sign, bits 2-1 exponent E, bit 0 mantissa m;
    E = 0 is subnormal, m/2; E > 0 is 2^(E-1) * (1 + m/2).  No NaN or inf.
    int [...] -> fp64 [...]."""
    c = np.asarray(code, dtype=np.int64)
    E = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    mag = np.where(E == 0, m / 2.0, np.exp2(E - 1.0) * (1.0 + m / 2.0))
    return np.where(c & 8, -mag, mag)


def e8m0_scale(e) -> np.ndarray:
    """E8M0 block scale [GGUF, the MXFP4 dequant commit]: 2^(e - 127), and
    e = 0xFF is NaN.  uint8 [...] -> fp64 [...]."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.exp2(e - 127.0))


def dequant_mxfp4(blocks: np.ndarray) -> np.ndarray:
    """MXFP4 [GGUF, the MXFP4 dequant commit]: 17-byte blocks of 32 values,
    the E8M0 exponent byte then 16 bytes of 4-bit codes, low nibble first
    (element 2i is the low nibble of code byte i, element 2i+1 its high
    nibble); value = e2m1(code) * 2^(e - 127).  Every product is exact in fp32
    (a 2-bit significand times a power of two, subnormals included) unless it
    exceeds fp32's range (e = 254 with |value| >= 2), where the fp32 result is
    +-inf.  blocks: uint8 [..., 17] -> fp32 [..., 32]."""
    e = blocks[..., 0]
    b = blocks[..., 1:17].astype(np.int64)
    codes = np.stack([b & 15, b >> 4], axis=-1).reshape(b.shape[:-1] + (32,))
    with np.errstate(invalid="ignore", over="ignore"):
        return (e2m1_value(codes) * e8m0_scale(e)[..., None]).astype(np.float32)


def e4m3_value(byte) -> np.ndarray:
    """FP8 E4M3 [GGUF, the DSv4 FP8 block dequant commit]: bit 7 sign, bits
    6-3 exponent with bias 7, bits 2-0 mantissa; exponent 0 is subnormal
    (m/8 * 2^-6); 0x7F and 0xFF are NaN; the largest magnitude is 448.
    uint8 [...] -> fp64 [...]."""
    b = np.asarray(byte, dtype=np.int64)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, np.exp2(e - 7.0) * (1.0 + m / 8.0))
    v = np.where(b & 0x80, -mag, mag)
    return np.where((b & 0x7F) == 0x7F, np.nan, v)


def dequant_fp8_block(w: np.ndarray, scales: np.ndarray, row_block: int = 128) -> np.ndarray:
    """FP8 block weights [GGUF, the DSv4 FP8 block dequant commit]: one E4M3
    byte per weight and one fp32 scale per 128 x 128 block;
    out[i, j] = e4m3(w[i, j]) * scales[i/128, j/128], the product rounded once
    in fp32.  w uint8 [..., N, K], scales fp32 [..., N/row_block, K/128]
    (row_block 1: one scale row per weight row, for a selection of rows)
    -> fp32 [..., N, K]."""
    v = e4m3_value(w).astype(np.float32)        # exact: 4 significant bits
    s = np.repeat(np.repeat(np.asarray(scales, np.float32), row_block, axis=-2), 128, axis=-1)
    with np.errstate(invalid="ignore", over="ignore"):
        return (v * s).astype(np.float32)


def dequant(W) -> np.ndarray:
    """Whole weight tensor (a synth.QWeights) -> fp32 [E, N, K]."""
    if W.fmt == "int4":
        return dequant_int4(W.qs, W.scale, W.bias, W.group)
    if W.fmt == "fp8":
        return dequant_fp8_block(W.qs, W.scale, W.group)
    if W.fmt == "q8_0":
        v = dequant_q8_0(W.blocks)
    elif W.fmt == "q2_k":
        v = dequant_q2_k(W.blocks)
    elif W.fmt == "iq2_xxs":
        v = dequant_iq2_xxs(W.blocks, W.grid)
    elif W.fmt == "mxfp4":
        v = dequant_mxfp4(W.blocks)
    elif W.fmt == "q4_k":
        v = dequant_q4_k(W.blocks)
    elif W.fmt == "q6_k":
        v = dequant_q6_k(W.blocks)
    else:
        raise ValueError(W.fmt)
    return v.reshape(W.E, W.N, W.K)


def dequant_rows(W, e: int, rows) -> np.ndarray:
    """fp32 [len(rows), K] for expert e's given output rows."""
    return dequant(W.expert_rows(e, rows))[0]


# ---------------------------------------------------------------------------
# matmuls
# ---------------------------------------------------------------------------

def qmm(x64: np.ndarray, W, e: int = 0) -> np.ndarray:
    """Dense quantised matmul [SHIM dense qmm cell]: y = x . W[e]^T in fp64.
    x64: fp64 [M, K]."""
    return x64 @ dequant(W)[e].astype(np.float64).T


def silu(z):
    """silu(z) = z / (1 + exp(-z)) in fp64 [BAGEL fused swiglu commit]."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def plan(ids: np.ndarray, n_experts: int, bm: int):
    """Expert-sorted routing plan [DSV4 PR body: the map0 work queue that
    feeds tiles of routed tokens to the MoE prefill GEMM].

    Pair p = t*k + j of ids[T, k].  Pairs whose id is outside [0, E) are dropped
    and counted.  Pairs are listed expert by expert, ascending pair id within an
    expert; each expert's run is cut into tiles of at most `bm` rows.
    Returns dict(dropped, counts[E], offsets[E+1], sorted[P_valid],
    tiles[n_tiles, 3] of (expert, row0, nrows))."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < n_experts)
    counts = np.zeros(n_experts, dtype=np.int64)
    buckets: list[list[int]] = [[] for _ in range(n_experts)]
    for p in np.nonzero(valid)[0]:
        buckets[flat[p]].append(int(p))
        counts[flat[p]] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_ = np.array([p for b in buckets for p in b], dtype=np.int64)
    tiles = []
    for e in range(n_experts):
        for r in range(0, int(counts[e]), bm):
            tiles.append((e, int(offsets[e]) + r, min(bm, int(counts[e]) - r)))
    return dict(dropped=int((~valid).sum()), counts=counts, offsets=offsets,
                sorted=sorted_, tiles=np.array(tiles, dtype=np.int64).reshape(-1, 3))


def _by_expert(ids: np.ndarray, E: int):
    flat = np.asarray(ids).reshape(-1)
    for e in range(E):
        pairs = np.nonzero(flat == e)[0]
        if len(pairs):
            yield e, pairs


def moe_gate_up(x64: np.ndarray, ids: np.ndarray, Wgu) -> np.ndarray:
    """Gate/up stage for every routed pair p = t*k + j, e = ids[t, j]:
    g = x_t . Wg[e]^T, u = x_t . Wu[e]^T (Wg = rows 0..I-1 and Wu = rows I..2I-1
    of the fused weight), h_p = silu(g) * u.  fp64 [P, I] in pair order."""
    T, k = ids.shape
    I = Wgu.N // 2
    h = np.zeros((T * k, I))
    for e, pairs in _by_expert(ids, Wgu.E):
        W = dequant_rows(Wgu, e, np.arange(Wgu.N)).astype(np.float64)
        gu = x64[pairs // k] @ W.T
        h[pairs] = silu(gu[:, :I]) * gu[:, I:]
    return h


def moe_down_combine(h64: np.ndarray, ids: np.ndarray, w: np.ndarray, Wd) -> np.ndarray:
    """Down stage plus weighted combine [DSV4 sum-folded q2_K down; BAGEL
    scalar-FMA top-K accumulator]: out_t = sum_j w[t,j] * (h_{t,j} . Wd[e]^T),
    j ascending.  h64 fp64 [P, I] in pair order -> fp64 [T, H]."""
    T, k = ids.shape
    y = np.zeros((T * k, Wd.N))
    for e, pairs in _by_expert(ids, Wd.E):
        W = dequant_rows(Wd, e, np.arange(Wd.N)).astype(np.float64)
        y[pairs] = h64[pairs] @ W.T
    return combine_pairs(y, ids, w, Wd.E)


def combine_pairs(y_pairs: np.ndarray, ids: np.ndarray, w: np.ndarray, n_experts: int) -> np.ndarray:
    """Top-k combine of per-pair expert outputs [BAGEL scalar-FMA top-K
    accumulator]: out_t = sum_j w[t,j] * y[t*k + j] over the pairs whose
    expert id is in [0, E); j ascending.  y fp64 [T*k, N] in pair order."""
    T, k = ids.shape
    y = np.asarray(y_pairs, np.float64).reshape(T, k, -1)
    ok = (ids >= 0) & (ids < n_experts)
    out = np.zeros((T, y.shape[2]))
    for j in range(k):
        out += np.where(ok[:, j, None], np.asarray(w, np.float64)[:, j, None] * y[:, j], 0.0)
    return out


def moe_ffn(x64, ids, w, Wgu, Wd, h_dtype: str | None = None, shared=None, shared_gate=None,
            residual=None):
    """Whole MoE FFN.  If h_dtype is given, h is rounded to that storage dtype
    between the two GEMMs (the storage point of the GPU path).  `shared` is an
    optional (gate_up, down) pair of dense weights, added with weight 1 or,
    with per-token gate logits `shared_gate`, with weight sigmoid(logit);
    `residual` is added last (see gated_shared_residual)."""
    h = moe_gate_up(x64, ids, Wgu)
    if h_dtype is not None:
        h = out_to_f64(round_out(h, h_dtype), h_dtype)
    out = moe_down_combine(h, ids, w, Wd)
    if shared is not None:
        sgu, sd = shared
        I = sgu.N // 2
        gu = qmm(x64, sgu)
        hs = silu(gu[:, :I]) * gu[:, I:]
        if h_dtype is not None:
            hs = out_to_f64(round_out(hs, h_dtype), h_dtype)
        return gated_shared_residual(out, qmm(hs, sd), shared_gate, residual)
    return gated_shared_residual(out, None, None, residual)


def gated_shared_residual(moe_out, shared_out=None, gate_logits=None, residual=None):
    """Post-MoE epilogue [BAGEL, the commit adding the scalar-FMA wrappers:
    the sigmoid-gated FMA with the residual add folded in]:
        out = residual + sigmoid(g_t) * shared + moe_out
    per token t, every term optional (a missing gate means weight 1).  fp64."""
    out = np.array(moe_out, dtype=np.float64)
    if shared_out is not None:
        g = 1.0
        if gate_logits is not None:
            with np.errstate(over="ignore"):  # exp(-g) = inf for g << 0 gives the exact limit 0
                g = (1.0 / (1.0 + np.exp(-np.asarray(gate_logits, np.float64))))[:, None]
        out = out + g * np.asarray(shared_out, np.float64)
    if residual is not None:
        out = out + np.asarray(residual, np.float64)
    return out


def moe_gate_up_rows(x64, ids, Wgu, pairs, cols) -> np.ndarray:
    """h[p, c] for selected pairs and columns only (for full-size sampling)."""
    k = ids.shape[1]
    I = Wgu.N // 2
    cols = np.asarray(cols)
    out = np.zeros((len(pairs), len(cols)))
    for i, p in enumerate(pairs):
        e = int(ids.reshape(-1)[p])
        W = dequant_rows(Wgu, e, np.concatenate([cols, cols + I])).astype(np.float64)
        gu = W @ x64[p // k]
        out[i] = silu(gu[:len(cols)]) * gu[len(cols):]
    return out


def moe_down_rows(h64_pairs: dict, ids, w, Wd, tokens, cols) -> np.ndarray:
    """out[t, c] for selected tokens and columns; h64_pairs maps pair id ->
    fp64 [I] (the h the down stage consumed)."""
    k = ids.shape[1]
    cols = np.asarray(cols)
    out = np.zeros((len(tokens), len(cols)))
    for i, t in enumerate(tokens):
        for j in range(k):
            e = int(ids[t, j])
            W = dequant_rows(Wd, e, cols).astype(np.float64)
            out[i] += np.float64(w[t, j]) * (W @ h64_pairs[t * k + j])
    return out


# ---------------------------------------------------------------------------
# routers (the step before the path: logits -> expert ids and top-k weights)
# ---------------------------------------------------------------------------

def router_topk_softmax(logits: np.ndarray, k: int, bias: np.ndarray | None = None):
    """Softmax top-k router [BAGEL, the commit moving the MoE router top-K to
    the GPU: per row the k largest logits, weights from a softmax over the
    selected logits, summing to 1; it replaces a CPU top-K + softmax].

    Without a bias the selection compares the logits themselves (no
    arithmetic), equal logits going to the lower expert index.

    With a per-expert bias [BAGEL, the LFM2-MoE softmax-then-bias routing and
    the fix that makes the router apply it]: p = softmax over all experts, the
    k largest p_e + bias_e are selected, and the weights are the selected
    p renormalised to sum 1 (reading: the same weights as the unbiased router
    gives for the same selection).  The selection is decided in fp32 (p and
    p + bias formed in fp32); the weights use fp64 p.

    Returns ids int32 [T, k] (best first), w float64 [T, k]."""
    L = np.asarray(logits, dtype=np.float64)
    if bias is None:
        order = np.argsort(-L, axis=1, kind="stable")[:, :k]   # stable: ties keep index order
        sel = np.take_along_axis(L, order, axis=1)
        z = np.exp(sel - sel.max(axis=1, keepdims=True))
        return order.astype(np.int32), z / z.sum(axis=1, keepdims=True)
    biased = router_softmax_bias_scores(L, bias)
    order = np.argsort(-biased.astype(np.float64), axis=1, kind="stable")[:, :k]
    p64 = np.exp(L - L.max(axis=1, keepdims=True))
    sel = np.take_along_axis(p64, order, axis=1)
    return order.astype(np.int32), sel / sel.sum(axis=1, keepdims=True)


def router_softmax_bias_scores(logits: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """Selection scores of the softmax-then-bias router in fp32: p + bias with
    p = exp(l - max l) / sum exp(l - max l) over the row.  fp32 [T, E]."""
    L32 = np.asarray(logits, dtype=np.float32)
    e32 = np.exp(L32 - L32.max(axis=1, keepdims=True))
    p32 = (e32 / e32.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return (p32 + np.asarray(bias, np.float32)[None, :]).astype(np.float32)


def _softplus_f32(x: np.ndarray) -> np.ndarray:
    """softplus(x) = max(x, 0) + log(1 + exp(-|x|)) evaluated in fp32 [GGUF,
    the DeepSeek V4 routing scoring commit: the stable form, since
    log(1 + exp(x)) overflows for large x]."""
    x = np.asarray(x, dtype=np.float32)
    return (np.maximum(x, np.float32(0)) + np.log1p(np.exp(-np.abs(x)))).astype(np.float32)


def router_sqrtsoftplus(logits: np.ndarray, bias: np.ndarray, k: int, scale: float):
    """DSv4 router [GGUF, the DeepSeek V4 routing scoring commit]:
    unbiased score s_e = sqrt(softplus(l_e)); the k largest biased scores
    s_e + bias_e are selected (aux-loss-free load balancing); the gather
    weight of a selected expert is s_e * routed_scaling_factor.

    The selection is an argmax decided in the kernel's precision: s and
    s + bias are formed in fp32 from fp32 logits (equal biased scores go to
    the lower expert index).  Weights use the fp64 score.
    Returns ids int32 [T, k], w float64 [T, k], biased fp32 scores [T, E]."""
    L32 = np.asarray(logits, dtype=np.float32)
    s32 = np.sqrt(_softplus_f32(L32)).astype(np.float32)
    biased = (s32 + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    order = np.argsort(-biased.astype(np.float64), axis=1, kind="stable")[:, :k]
    L64 = np.take_along_axis(L32.astype(np.float64), order, axis=1)
    sp64 = np.maximum(L64, 0.0) + np.log1p(np.exp(-np.abs(L64)))
    return order.astype(np.int32), np.sqrt(sp64) * float(scale), biased

"""Python binding of libqmoe (the block-quantized MoE expert matmul for MI355X).

Argument marshalling only: every step runs in the HIP kernels of libqmoe.so,
called through its C ABI (include/qmoe.h).  PyTorch provides device memory and
the current stream.  There is no fallback: if the library is missing, or the
device is not gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmoe.so")

# enums mirrored from include/qmoe.h
F32, F16, BF16 = 0, 1, 2
Q8_0, Q2_K, IQ2_XXS, INT4, MXFP4, FP8, Q4_K, Q6_K = 0, 1, 2, 3, 4, 5, 6, 7
EPI_STORE, EPI_SWIGLU, EPI_WEIGHTED_COMBINE, EPI_ACCUMULATE = 0, 1, 2, 3
A_GATHER_TOKENS, A_SORTED_ROWS = 0, 1
ROUTER_SOFTMAX, ROUTER_SQRTSOFTPLUS = 0, 1
FORMATS = {"q8_0": Q8_0, "q2_k": Q2_K, "iq2_xxs": IQ2_XXS, "int4": INT4, "mxfp4": MXFP4, "fp8": FP8,
           "q4_k": Q4_K, "q6_k": Q6_K}
MAX_TOPK, MAX_EXPERTS, MAX_GEMV_BATCH = 8, 1024, 64


class QmoeError(RuntimeError):
    pass


class _Weights(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("group", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("qs", ctypes.c_void_p), ("aux", ctypes.c_void_p),
        ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p),
        ("d", ctypes.c_void_p), ("dmin", ctypes.c_void_p),
        ("grid", ctypes.c_void_p), ("signs", ctypes.c_void_p),
    ]


_lib = None

_SIGS = {
    "qmoe_split_q8_0": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p],
    "qmoe_split_q2_k": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 4,
    "qmoe_split_iq2_xxs": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 2,
    "qmoe_split_mxfp4": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 2,
    "qmoe_split_q4_k": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 4,
    "qmoe_split_q6_k": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 4,
    "qmoe_dequant_q4_k": [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                                  ctypes.c_void_p],
    "qmoe_dequant_q6_k": [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                                  ctypes.c_void_p],
    "qmoe_dequant_mxfp4": [ctypes.c_void_p] * 2 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                                    ctypes.c_void_p],
    "qmoe_split_fp8": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p],
    "qmoe_dequant_fp8": [ctypes.c_void_p] * 2 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                                  ctypes.c_void_p],
    "qmoe_split_int4": [ctypes.c_void_p] * 3 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p],
    "qmoe_iq2_signs_table": [ctypes.c_void_p],
    "qmoe_dequant_q8_0": [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                          ctypes.c_int32, ctypes.c_void_p],
    "qmoe_dequant_q2_k": [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                                  ctypes.c_void_p],
    "qmoe_dequant_iq2_xxs": [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                                     ctypes.c_void_p],
    "qmoe_dequant_int4": [ctypes.c_void_p] * 2 + [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "qmoe_qmm_dense": [ctypes.POINTER(_Weights), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "qmoe_plan_bytes": [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32],
    "qmoe_moe_plan": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p],
    "qmoe_moe_gather_qmm": [ctypes.POINTER(_Weights), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "qmoe_moe_combine": [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "qmoe_moe_combine_shared": [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "qmoe_combine_cast": [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "qmoe_moe_gemv": [ctypes.POINTER(_Weights), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "qmoe_router_topk": [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p,
                         ctypes.c_void_p],
    "qmoe_check_device": [],
    "qmoe_strerror": [ctypes.c_int],
    "qmoe_split_rows": [ctypes.c_int64],
    "qmoe_moe_gather_qmm_combine_static": [ctypes.POINTER(_Weights), ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p],
    "qmoe_static_acc_bytes": [],
    "qmoe_workspace_bytes": [ctypes.c_int32, ctypes.POINTER(_Weights), ctypes.c_int64, ctypes.c_int32, ctypes.c_int32],
}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded libqmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QmoeError(f"libqmoe.so not built ({LIB_PATH}); run python -m block_quantized_moe_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.qmoe_plan_bytes.restype = ctypes.c_size_t
        L.qmoe_workspace_bytes.restype = ctypes.c_size_t
        L.qmoe_split_rows.restype = ctypes.c_int64
        L.qmoe_static_acc_bytes.restype = ctypes.c_size_t
        L.qmoe_strerror.restype = ctypes.c_char_p
        L.qmoe_iq2_signs_table.restype = None
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise QmoeError(f"{what}: {lib().qmoe_strerror(status).decode()} ({status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _np_ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------------------
# host-side split (C functions of the library)
# ---------------------------------------------------------------------------

def split_rows(rows: int) -> int:
    """Rows of every tiled split array: rows rounded up to a multiple of 16."""
    return int(lib().qmoe_split_rows(rows))


def split_q8_0(aos: np.ndarray, rows: int, k: int):
    """Q8_0 blocks [rows, k/32, 34] -> tiled (codes, scales), sized for split_rows(rows)."""
    aos = np.ascontiguousarray(aos, dtype=np.uint8).reshape(-1)
    if aos.size != rows * (k // 32) * 34:
        raise QmoeError("split_q8_0: block count does not match rows/k")
    R = split_rows(rows)
    qs = np.empty(R * k, np.int8)
    d = np.empty(R * (k // 32), np.uint16)
    _check(lib().qmoe_split_q8_0(_np_ptr(aos), rows, k, _np_ptr(qs), _np_ptr(d)), "split_q8_0")
    return qs, d


def split_q2_k(aos: np.ndarray, rows: int, k: int):
    """Q2_K blocks [rows, k/256, 84] -> tiled (qs bytes, scales, d, dmin)."""
    aos = np.ascontiguousarray(aos, dtype=np.uint8).reshape(-1)
    if aos.size != rows * (k // 256) * 84:
        raise QmoeError("split_q2_k: block count does not match rows/k")
    nb = split_rows(rows) * (k // 256)
    qs = np.empty(nb * 16, np.uint32)
    sc = np.empty(nb * 16, np.uint8)
    d = np.empty(nb, np.uint16)
    dmin = np.empty(nb, np.uint16)
    _check(lib().qmoe_split_q2_k(_np_ptr(aos), rows, k, _np_ptr(qs), _np_ptr(sc), _np_ptr(d), _np_ptr(dmin)),
           "split_q2_k")
    return qs, sc, d, dmin


def split_q4_k(aos: np.ndarray, rows: int, k: int):
    """Q4_K blocks [rows, k/256, 144] -> tiled (qs bytes, scales|mins bytes, d, dmin)."""
    aos = np.ascontiguousarray(aos, dtype=np.uint8).reshape(-1)
    if aos.size != rows * (k // 256) * 144:
        raise QmoeError("split_q4_k: block count does not match rows/k")
    nb = split_rows(rows) * (k // 256)
    qs = np.empty(nb * 128, np.uint8)
    sc = np.empty(nb * 16, np.uint8)
    d = np.empty(nb, np.uint16)
    dmin = np.empty(nb, np.uint16)
    _check(lib().qmoe_split_q4_k(_np_ptr(aos), rows, k, _np_ptr(qs), _np_ptr(sc), _np_ptr(d), _np_ptr(dmin)),
           "split_q4_k")
    return qs, sc, d, dmin


def split_q6_k(aos: np.ndarray, rows: int, k: int):
    """Q6_K blocks [rows, k/256, 210] -> tiled (low-nibble bytes, top-bit-pair bytes, int8 scales, d)."""
    aos = np.ascontiguousarray(aos, dtype=np.uint8).reshape(-1)
    if aos.size != rows * (k // 256) * 210:
        raise QmoeError("split_q6_k: block count does not match rows/k")
    nb = split_rows(rows) * (k // 256)
    qs = np.empty(nb * 128, np.uint8)
    qh = np.empty(nb * 64, np.uint8)
    sc = np.empty(nb * 16, np.int8)
    d = np.empty(nb, np.uint16)
    _check(lib().qmoe_split_q6_k(_np_ptr(aos), rows, k, _np_ptr(qs), _np_ptr(qh), _np_ptr(sc), _np_ptr(d)),
           "split_q6_k")
    return qs, qh, sc, d


def split_iq2_xxs(aos: np.ndarray, rows: int, k: int):
    """IQ2_XXS blocks [rows, k/256, 66] -> tiled ((index, aux) word pairs, d)."""
    aos = np.ascontiguousarray(aos, dtype=np.uint8).reshape(-1)
    if aos.size != rows * (k // 256) * 66:
        raise QmoeError("split_iq2_xxs: block count does not match rows/k")
    nb = split_rows(rows) * (k // 256)
    ia = np.empty(nb * 16, np.uint32)
    d = np.empty(nb, np.uint16)
    _check(lib().qmoe_split_iq2_xxs(_np_ptr(aos), rows, k, _np_ptr(ia), _np_ptr(d)), "split_iq2_xxs")
    return ia, d


def split_mxfp4(aos: np.ndarray, rows: int, k: int):
    """MXFP4 blocks [rows, k/32, 17] -> tiled (code words, E8M0 exponents)."""
    aos = np.ascontiguousarray(aos, dtype=np.uint8).reshape(-1)
    if aos.size != rows * (k // 32) * 17:
        raise QmoeError("split_mxfp4: block count does not match rows/k")
    R = split_rows(rows)
    qs = np.empty(R * k // 8, np.uint32)
    e = np.empty(R * (k // 32), np.uint8)
    _check(lib().qmoe_split_mxfp4(_np_ptr(aos), rows, k, _np_ptr(qs), _np_ptr(e)), "split_mxfp4")
    return qs, e


def split_fp8(w: np.ndarray, rows: int, k: int):
    """FP8 E4M3 codes [rows, k] -> tiled codes (the fp32 block scales need no split)."""
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    if w.size != rows * k:
        raise QmoeError("split_fp8: code count does not match rows/k")
    qs = np.empty(rows * k, np.uint8)
    _check(lib().qmoe_split_fp8(_np_ptr(w), rows, k, _np_ptr(qs)), "split_fp8")
    return qs


def split_int4(words: np.ndarray, scale: np.ndarray, bias: np.ndarray, rows: int, k: int, group: int):
    """MLX-style int4 rows -> (tiled code words, packed scale|bias<<16 words)."""
    words = np.ascontiguousarray(words, dtype=np.uint32).reshape(-1)
    scale = np.ascontiguousarray(scale, dtype=np.uint16).reshape(-1)
    bias = np.ascontiguousarray(bias, dtype=np.uint16).reshape(-1)
    if words.size != rows * (k // 8) or scale.size != rows * (k // max(group, 1)) or bias.size != scale.size:
        raise QmoeError("split_int4: array sizes do not match rows/k/group")
    R = split_rows(rows)
    qs = np.empty(R * (k // 8), np.uint32)
    sb = np.empty(R * (k // max(group, 1)), np.uint32)
    _check(lib().qmoe_split_int4(_np_ptr(words), _np_ptr(scale), _np_ptr(bias), rows, k, group,
                                 _np_ptr(qs), _np_ptr(sb)), "split_int4")
    return qs, sb


def iq2_signs_table() -> np.ndarray:
    out = np.zeros(128, np.uint8)
    lib().qmoe_iq2_signs_table(_np_ptr(out))
    return out


# ---------------------------------------------------------------------------
# device weights
# ---------------------------------------------------------------------------

@dataclass
class DeviceWeights:
    """A stacked expert weight tensor in its GPU-resident split form."""
    fmt: str
    E: int
    N: int
    K: int
    group: int = 0
    tensors: dict = field(default_factory=dict)

    def struct(self) -> _Weights:
        t = self.tensors
        return _Weights(FORMATS[self.fmt], self.E, self.N, self.K, self.group, 0,
                        _ptr(t.get("qs")), _ptr(t.get("aux")), _ptr(t.get("scales")),
                        _ptr(t.get("biases")), _ptr(t.get("d")), _ptr(t.get("dmin")),
                        _ptr(t.get("grid")), _ptr(t.get("signs")))

    @property
    def nbytes(self) -> int:
        return int(sum(v.numel() * v.element_size() for k, v in self.tensors.items() if k not in ("grid", "signs")))

    def clone(self) -> "DeviceWeights":
        return DeviceWeights(self.fmt, self.E, self.N, self.K, self.group,
                             {k: (v if k in ("grid", "signs") else v.clone()) for k, v in self.tensors.items()})


def _dev(a: np.ndarray, device):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def upload(fmt: str, E: int, N: int, K: int, *, device="cuda", blocks=None, qs=None, scale=None,
           bias=None, group: int = 0, grid=None) -> DeviceWeights:
    """Split on-disk weights on the host (library splitter) and copy them to the device.

    blocks: uint8 on-disk blocks [E, N, K/block, bytes] for q8_0 / q2_k / iq2_xxs / mxfp4 / q4_k / q6_k.
    qs, scale, bias: MLX-style int4 arrays for int4; for fp8, qs uint8 E4M3 codes
    [E, N, K] and scale fp32 [E, N/128, K/128].  grid: uint8 [256, 8] (iq2_xxs)."""
    t = {}
    if fmt == "q8_0":
        q, d = split_q8_0(blocks, E * N, K)
        t["qs"], t["scales"] = _dev(q, device), _dev(d, device)
    elif fmt == "q2_k":
        q, sc, d, dmin = split_q2_k(blocks, E * N, K)
        t["qs"], t["scales"], t["d"], t["dmin"] = (_dev(q, device), _dev(sc, device), _dev(d, device), _dev(dmin, device))
    elif fmt == "iq2_xxs":
        ia, d = split_iq2_xxs(blocks, E * N, K)
        t["qs"], t["d"] = _dev(ia, device), _dev(d, device)
        t["grid"] = _dev(np.ascontiguousarray(grid, np.uint8).reshape(-1), device)
        t["signs"] = _dev(iq2_signs_table(), device)
    elif fmt == "mxfp4":
        q, e = split_mxfp4(blocks, E * N, K)
        t["qs"], t["scales"] = _dev(q, device), _dev(e, device)
    elif fmt == "q4_k":
        q, sc, d, dmin = split_q4_k(blocks, E * N, K)
        t["qs"], t["scales"], t["d"], t["dmin"] = (_dev(q, device), _dev(sc, device), _dev(d, device), _dev(dmin, device))
    elif fmt == "q6_k":
        q, qh, sc, d = split_q6_k(blocks, E * N, K)
        t["qs"], t["aux"], t["scales"], t["d"] = (_dev(q, device), _dev(qh, device), _dev(sc, device), _dev(d, device))
    elif fmt == "fp8":
        t["qs"] = _dev(split_fp8(qs, E * N, K), device)
        t["scales"] = _dev(np.ascontiguousarray(scale, np.float32).reshape(-1), device)
    elif fmt == "int4":
        q, sb = split_int4(qs, scale, bias, E * N, K, group)
        t["qs"], t["scales"] = _dev(q, device), _dev(sb, device)
    else:
        raise ValueError(fmt)
    return DeviceWeights(fmt, E, N, K, group, t)


# ---------------------------------------------------------------------------
# compute entry points (same names as the C ABI, without the qmoe_ prefix)
# ---------------------------------------------------------------------------

_TORCH_DT = {}


def _dt(code):
    import torch
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[code]


def _code(t):
    import torch
    return {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[t.dtype]


def _need(t, name, *, shape=None, cols=None, min_rows=None, dtypes=None, dim=None):
    """Check a caller-supplied tensor before its pointer reaches the library:
    contiguity, rank, shape (None entries match anything), dtype, and that it
    is on a GPU.  Raises ValueError."""
    import torch
    if t is None:
        raise ValueError(f"{name}: a tensor is required")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name}: expected {dim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and (t.dim() != len(shape) or any(w is not None and int(v) != int(w)
                                                           for v, w in zip(t.shape, shape))):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if cols is not None and (t.dim() < 1 or int(t.shape[-1]) != int(cols)):
        raise ValueError(f"{name}: expected {cols} columns, got shape {tuple(t.shape)}")
    if min_rows is not None and (t.dim() < 1 or int(t.shape[0]) < int(min_rows)):
        raise ValueError(f"{name}: expected at least {min_rows} rows, got shape {tuple(t.shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")


def _acts():
    import torch
    return (torch.float16, torch.bfloat16)


def _outs():
    import torch
    return (torch.float32, torch.float16, torch.bfloat16)


def check_device():
    _check(lib().qmoe_check_device(), "check_device")


def dequant(w: DeviceWeights, out_dtype: int = F32, out=None):
    """Whole weight tensor -> dense [E, N, K] on the device (bit-exact)."""
    import torch
    if out is None:
        out = torch.empty((w.E, w.N, w.K), dtype=_dt(out_dtype), device=w.tensors["qs"].device)
    _need(out, "out", shape=(w.E, w.N, w.K), dtypes=_outs())
    if _code(out) != out_dtype:
        raise ValueError(f"out: dtype {out.dtype} does not match out_dtype {out_dtype}")
    t = w.tensors
    L = lib()
    s = _stream()
    if w.fmt == "q8_0":
        st = L.qmoe_dequant_q8_0(_ptr(t["qs"]), _ptr(t["scales"]), w.E * w.N, w.K, _ptr(out), out_dtype, s)
    elif w.fmt == "q2_k":
        st = L.qmoe_dequant_q2_k(_ptr(t["qs"]), _ptr(t["scales"]), _ptr(t["d"]), _ptr(t["dmin"]),
                                 w.E * w.N, w.K, _ptr(out), out_dtype, s)
    elif w.fmt == "iq2_xxs":
        st = L.qmoe_dequant_iq2_xxs(_ptr(t["qs"]), _ptr(t["d"]), _ptr(t["grid"]), _ptr(t["signs"]),
                                    w.E * w.N, w.K, _ptr(out), out_dtype, s)
    elif w.fmt == "fp8":
        st = L.qmoe_dequant_fp8(_ptr(t["qs"]), _ptr(t["scales"]), w.E * w.N, w.K, _ptr(out), out_dtype, s)
    elif w.fmt == "mxfp4":
        st = L.qmoe_dequant_mxfp4(_ptr(t["qs"]), _ptr(t["scales"]), w.E * w.N, w.K, _ptr(out), out_dtype, s)
    elif w.fmt == "q4_k":
        st = L.qmoe_dequant_q4_k(_ptr(t["qs"]), _ptr(t["scales"]), _ptr(t["d"]), _ptr(t["dmin"]),
                                 w.E * w.N, w.K, _ptr(out), out_dtype, s)
    elif w.fmt == "q6_k":
        st = L.qmoe_dequant_q6_k(_ptr(t["qs"]), _ptr(t["aux"]), _ptr(t["scales"]), _ptr(t["d"]),
                                 w.E * w.N, w.K, _ptr(out), out_dtype, s)
    else:
        st = L.qmoe_dequant_int4(_ptr(t["qs"]), _ptr(t["scales"]), w.E * w.N, w.K, w.group,
                                 _ptr(out), out_dtype, s)
    _check(st, f"dequant_{w.fmt}")
    return out


def qmm_dense(w: DeviceWeights, x, epilogue: int = EPI_STORE, out_dtype: int = F16, out=None):
    import torch
    _need(x, "x", dim=2, cols=w.K, dtypes=_acts())
    M = x.shape[0]
    n = w.N // 2 if epilogue == EPI_SWIGLU else w.N
    if out is None:
        out = torch.empty((M, n), dtype=_dt(out_dtype), device=x.device)
    _need(out, "out", shape=(M, n), dtypes=(torch.float32,) if epilogue == EPI_ACCUMULATE else _outs())
    ws = w.struct()
    _check(lib().qmoe_qmm_dense(ctypes.byref(ws), _ptr(x), _code(x), M, epilogue, _ptr(out), _code(out), _stream()),
           "qmm_dense")
    return out


def plan_bytes(t: int, topk: int, E: int, bm: int) -> int:
    return int(lib().qmoe_plan_bytes(t, topk, E, bm))


def moe_plan(ids, E: int, bm: int = 80, plan=None):
    import torch
    _need(ids, "ids", dim=2, dtypes=(torch.int32,))
    T, k = ids.shape
    nbytes = plan_bytes(T, k, E, bm)
    if plan is None:
        plan = torch.empty(nbytes // 4, dtype=torch.int32, device=ids.device)
    _need(plan, "plan", dtypes=(torch.int32,))
    if plan.numel() * 4 < nbytes:
        raise ValueError(f"plan: {plan.numel() * 4} bytes, the call needs {nbytes}")
    _check(lib().qmoe_moe_plan(_ptr(ids), T, k, E, bm, _ptr(plan), plan.numel() * 4, _stream()), "moe_plan")
    return plan


def router_topk(logits, k: int, scoring: int = ROUTER_SOFTMAX, bias=None, scale: float = 1.0,
                ids=None, weights=None):
    """Router top-k on the device: logits [T, E] (f32 / f16 / bf16) ->
    (ids int32 [T, k], weights f32 [T, k]), best first (include/qmoe.h)."""
    import torch
    _need(logits, "logits", dim=2, dtypes=_outs())
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _need(ids, "ids", shape=(T, k), dtypes=(torch.int32,))
    _need(weights, "weights", shape=(T, k), dtypes=(torch.float32,))
    if bias is not None:
        _need(bias, "bias", shape=(E,), dtypes=(torch.float32,))
    if T == 0:
        return ids, weights
    _check(lib().qmoe_router_topk(_ptr(logits), _code(logits), T, E, k, scoring, _ptr(bias), scale,
                                  _ptr(ids), _ptr(weights), _stream()), "router_topk")
    return ids, weights


def plan_views(plan, T: int, topk: int, E: int):
    """Named views of a plan buffer (layout in include/qmoe.h)."""
    P = T * topk
    counts = 8
    offsets = counts + E
    sorted_ = offsets + E + 1
    tiles = (sorted_ + P + 3) & ~3
    max_tiles16 = min(P, E) + P // 16
    inv = tiles + 4 * max_tiles16
    return dict(header=plan[:8], counts=plan[counts:counts + E], offsets=plan[offsets:offsets + E + 1],
                sorted=plan[sorted_:sorted_ + P], tiles=plan[tiles:tiles + 4 * max_tiles16].view(-1, 4),
                inv=plan[inv:inv + P])


def moe_gather_qmm(w: DeviceWeights, plan, T: int, topk: int, a, *, bm: int = 80,
                   a_mode: int = A_GATHER_TOKENS, topk_w=None, epilogue: int = EPI_STORE,
                   out_dtype: int = None, out=None, n_rows: int = None):
    """Gathered MoE matmul.  For STORE / SWIGLU the output has one row per
    sorted position (n_rows = number of valid pairs, default T * topk); with
    SORTED_ROWS the activations hold one row per sorted position.  Rows past
    the given tensors cannot be checked on the host (the plan's valid-pair
    count lives on the device): out and SORTED_ROWS activations must hold at
    least the plan's valid pairs."""
    import torch
    _need(a, "a", dim=2, cols=w.K, dtypes=_acts())
    if a_mode == A_GATHER_TOKENS and a.shape[0] != T:
        raise ValueError(f"a: GATHER_TOKENS takes [T={T}, K] activations, got {tuple(a.shape)}")
    if a_mode == A_SORTED_ROWS and n_rows is not None and a.shape[0] < n_rows:
        raise ValueError(f"a: {a.shape[0]} rows for {n_rows} valid pairs")
    _need(plan, "plan", dtypes=(torch.int32,))
    if plan.numel() * 4 < plan_bytes(T, topk, w.E, bm):
        raise ValueError("plan: smaller than a plan for this call")
    n = w.N // 2 if epilogue == EPI_SWIGLU else w.N
    rows = T * topk if n_rows is None else n_rows
    if out is None:
        if epilogue == EPI_WEIGHTED_COMBINE:
            out = torch.zeros((T, w.N), dtype=torch.float32, device=a.device)
        else:
            out = torch.empty((rows, n), dtype=_dt(out_dtype if out_dtype is not None else _code(a)), device=a.device)
    if epilogue == EPI_WEIGHTED_COMBINE:
        _need(out, "out", shape=(T, w.N), dtypes=(torch.float32,))
        _need(topk_w, "topk_w", shape=(T, topk), dtypes=(torch.float32,))
    else:
        _need(out, "out", dim=2, cols=n, min_rows=rows if n_rows is not None else 1, dtypes=_outs())
    ws = w.struct()
    _check(lib().qmoe_moe_gather_qmm(ctypes.byref(ws), _ptr(plan), T, topk, bm, _ptr(a), _code(a), a_mode,
                                     _ptr(topk_w), epilogue, _ptr(out), _code(out), _stream()), "moe_gather_qmm")
    return out


def _combine_checks(y, plan, T, topk, E, topk_w, out):
    import torch
    _need(y, "y", dim=2, dtypes=_outs())
    _need(plan, "plan", dtypes=(torch.int32,))
    if plan.numel() * 4 < plan_bytes(T, topk, E, 16):
        raise ValueError("plan: smaller than a plan for this call")
    _need(topk_w, "topk_w", shape=(T, topk), dtypes=(torch.float32,))
    _need(out, "out", shape=(T, y.shape[1]), dtypes=_outs())


def moe_gather_qmm_combine_static(w: DeviceWeights, plan, T: int, topk: int, a, topk_w, *, bm: int = 80,
                                  a_mode: int = A_SORTED_ROWS, out_dtype: int = BF16, out=None):
    """WEIGHTED_COMBINE gathered matmul plus the cast, with the fp32
    accumulator inside the library (no allocation in the call; include/qmoe.h)."""
    import torch
    _need(a, "a", dim=2, cols=w.K, dtypes=_acts())
    if a_mode == A_GATHER_TOKENS and a.shape[0] != T:
        raise ValueError(f"a: GATHER_TOKENS takes [T={T}, K] activations, got {tuple(a.shape)}")
    _need(plan, "plan", dtypes=(torch.int32,))
    if plan.numel() * 4 < plan_bytes(T, topk, w.E, bm):
        raise ValueError("plan: smaller than a plan for this call")
    _need(topk_w, "topk_w", shape=(T, topk), dtypes=(torch.float32,))
    if out is None:
        out = torch.empty((T, w.N), dtype=_dt(out_dtype), device=a.device)
    _need(out, "out", shape=(T, w.N), dtypes=_outs())
    ws = w.struct()
    _check(lib().qmoe_moe_gather_qmm_combine_static(ctypes.byref(ws), _ptr(plan), T, topk, bm, _ptr(a), _code(a),
                                                    a_mode, _ptr(topk_w), _ptr(out), _code(out), _stream()),
           "moe_gather_qmm_combine_static")
    return out


def moe_combine(y, plan, T: int, topk: int, E: int, topk_w, base=None, out_dtype: int = BF16, out=None):
    import torch
    N = y.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=_dt(out_dtype), device=y.device)
    _combine_checks(y, plan, T, topk, E, topk_w, out)
    if base is not None:
        _need(base, "base", shape=(T, N), dtypes=(torch.float32,))
    _check(lib().qmoe_moe_combine(_ptr(y), _code(y), _ptr(plan), T, topk, E, _ptr(topk_w), N, _ptr(base),
                                  _ptr(out), _code(out), _stream()), "moe_combine")
    return out


def moe_combine_shared(y, plan, T: int, topk: int, E: int, topk_w, shared=None, shared_gate=None,
                       residual=None, out_dtype: int = BF16, out=None):
    """Combine plus a sigmoid-gated shared expert and the residual add
    (include/qmoe.h); out may be the residual tensor itself."""
    import torch
    N = y.shape[1]
    if out is None:
        out = torch.empty((T, N), dtype=_dt(out_dtype), device=y.device)
    _combine_checks(y, plan, T, topk, E, topk_w, out)
    if shared is not None:
        _need(shared, "shared", shape=(T, N), dtypes=(torch.float32,))
    if shared_gate is not None:
        _need(shared_gate, "shared_gate", shape=(T,), dtypes=(torch.float32,))
    if residual is not None:
        _need(residual, "residual", shape=(T, N), dtypes=_outs())
    rcode = _code(residual) if residual is not None else F32
    _check(lib().qmoe_moe_combine_shared(_ptr(y), _code(y), _ptr(plan), T, topk, E, _ptr(topk_w), N, _ptr(shared),
                                         _ptr(shared_gate), _ptr(residual), rcode, _ptr(out), _code(out),
                                         _stream()), "moe_combine_shared")
    return out


def combine_cast(acc, out_dtype: int = BF16, out=None):
    import torch
    _need(acc, "acc", dtypes=(torch.float32,))
    if out is None:
        out = torch.empty(acc.shape, dtype=_dt(out_dtype), device=acc.device)
    _need(out, "out", shape=tuple(acc.shape), dtypes=_outs())
    _check(lib().qmoe_combine_cast(_ptr(acc), acc.numel(), _ptr(out), _code(out), _stream()), "combine_cast")
    return out


def moe_gemv(w: DeviceWeights, a, ids, topk_w=None, *, epilogue: int = EPI_SWIGLU,
             out_dtype: int = None, out=None):
    """Decode GEMV.  STORE/SWIGLU: a = x [B, K] -> [B, topk, N or N/2];
    WEIGHTED_COMBINE: a = h [B, topk, K] -> [B, N]."""
    import torch
    _need(ids, "ids", dim=2, dtypes=(torch.int32,))
    B, topk = ids.shape
    if epilogue == EPI_WEIGHTED_COMBINE:
        _need(a, "a", shape=(B, topk, w.K), dtypes=_acts())
        _need(topk_w, "topk_w", shape=(B, topk), dtypes=(torch.float32,))
    else:
        _need(a, "a", shape=(B, w.K), dtypes=_acts())
    od = out_dtype if out_dtype is not None else _code(a)
    n = w.N // 2 if epilogue == EPI_SWIGLU else w.N
    oshape = (B, w.N) if epilogue == EPI_WEIGHTED_COMBINE else (B, topk, n)
    if out is None:
        out = torch.empty(oshape, dtype=_dt(od), device=a.device)
    _need(out, "out", shape=oshape, dtypes=_outs())
    ws = w.struct()
    _check(lib().qmoe_moe_gemv(ctypes.byref(ws), _ptr(a), _code(a), B, _ptr(ids), _ptr(topk_w), topk, epilogue,
                               _ptr(out), _code(out), _stream()), "moe_gemv")
    return out

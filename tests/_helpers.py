"""Shared helpers of the GPU parity tests (marshalling and the error metric)."""
from __future__ import annotations

import numpy as np

import block_quantized_moe_amd as qm

CODES = {"f32": qm.F32, "f16": qm.F16, "bf16": qm.BF16}


def torch_act(bits: np.ndarray, dtype: str, device="cuda"):
    """uint16 bit patterns -> a torch fp16/bf16 tensor on the device."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).to(device)


def to_bits(t) -> np.ndarray:
    """A torch fp16/bf16 tensor -> uint16 bit patterns (host)."""
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def to_f64(t, dtype: str | None = None) -> np.ndarray:
    import torch
    if t.dtype == torch.float32:
        return t.detach().cpu().numpy().astype(np.float64)
    bits = to_bits(t)
    u = bits.astype(np.uint32)
    if t.dtype == torch.bfloat16:
        return (u << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def upload(W, device="cuda") -> "qm.DeviceWeights":
    if W.fmt == "int4":
        return qm.upload("int4", W.E, W.N, W.K, device=device, qs=W.qs, scale=W.scale, bias=W.bias, group=W.group)
    if W.fmt == "fp8":
        return qm.upload("fp8", W.E, W.N, W.K, device=device, qs=W.qs, scale=W.scale)
    return qm.upload(W.fmt, W.E, W.N, W.K, device=device, blocks=W.blocks, grid=W.grid)


def half_ulp(y: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of the output format at |y| (0 for fp32)."""
    if dtype == "f32":
        return np.zeros_like(y)
    mant, emin = (7, -126) if dtype == "bf16" else (10, -14)
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return 0.5 * np.exp2(e - mant)


def normwise_err(y: np.ndarray, r: np.ndarray, dtype: str) -> float:
    """max_i max(0, |y_i - r_i| - ulp_out(y_i)/2) / max_i |r_i| -- the relative
    error net of the unavoidable final rounding to the output dtype."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    num = np.maximum(0.0, np.abs(y - r) - half_ulp(y, dtype)).max(initial=0.0)
    den = np.abs(r).max(initial=0.0)
    return float(num / den) if den > 0 else float(num)


def report(y, r) -> dict:
    y = np.asarray(y, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    cos = float(y @ r / (np.linalg.norm(y) * np.linalg.norm(r) + 1e-300))
    return dict(max_rel=float(np.abs(y - r).max() / (np.abs(r).max() + 1e-300)),
                fro_rel=float(np.linalg.norm(y - r) / (np.linalg.norm(r) + 1e-300)), cosine=cos)


TOL = 2e-3  # normwise relative error bound on fp16 / bf16 outputs vs the fp64 oracle

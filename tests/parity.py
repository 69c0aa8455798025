"""Helpers shared by the GPU parity tests: device transfer of raw 16-bit
patterns and the comparison rules.

Comparison rules for c = B @ a in fp16/bf16 with an fp32 sum:
  * grading tolerance  |c_gpu - c_ref| <= 4e-3 * sum_j |B_ij a_j| + ulp(c_ref)
  * strict bound       |c_gpu - c_ref| <= ulp + 2^-24 * (ceil(k/64) + 8 + S) * sum_j |B_ij a_j|
    (S = k-splits).  Each lane adds its products serially into two
    accumulators -- at most ceil(k/128) terms each -- and a 6-level tree and
    the split combine follow, so every product passes through at most
    ceil(k/64) + 8 + S fp32 roundings; ulp covers the two roundings to the
    16-bit output (GPU and oracle), taken at the larger of the two results.
  * special values compare by class: NaN <-> NaN, +-inf <-> the same inf;
    zeros compare by value (+0 == -0).
"""
import math

import numpy as np
import torch

import oracle
from gemv_inputs import BF16, F16, torch_dtype

GRADE_REL = 4e-3
FP32_U = 2.0 ** -24


def to_device(bits: np.ndarray, dtype: int, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch_dtype(dtype))


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ulp(dtype: int, x: np.ndarray) -> np.ndarray:
    """Spacing of the dtype's values at |x| (subnormal spacing below the
    smallest normal)."""
    fb, emin = (10, -14) if dtype == F16 else (7, -126)
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - fb).astype(np.int64))


def compare(dtype, c_gpu_bits, c_ref_bits, absum, k, splits=1):
    """Return (ok_grade, ok_strict, max_grade_ratio, max_strict_ratio, first_bad)."""
    g = oracle.decode(dtype, c_gpu_bits)
    r = oracle.decode(dtype, c_ref_bits)
    gn, rn = np.isnan(g), np.isnan(r)
    gi, ri = np.isinf(g), np.isinf(r)
    cls_ok = (gn == rn) & (np.where(ri | gi, g == r, True) | rn)
    fin = np.isfinite(g) & np.isfinite(r)
    diff = np.abs(g - r)
    u = ulp(dtype, np.maximum(np.abs(np.where(fin, g, 0)), np.abs(np.where(fin, r, 0))))
    grade = GRADE_REL * absum + ulp(dtype, np.where(fin, r, 0))
    strict = u + FP32_U * (math.ceil(k / 64) + 8 + splits) * absum
    ok_g = cls_ok & (~fin | (diff <= grade))
    ok_s = cls_ok & (~fin | (diff <= strict))
    with np.errstate(divide="ignore", invalid="ignore"):
        rg = np.where(fin, diff / grade, 0.0)
        rs = np.where(fin, diff / strict, 0.0)
    bad = np.nonzero(~ok_s)[0]
    first = None
    if bad.size:
        i = int(bad[0])
        first = dict(row=i, gpu=float(g[i]), ref=float(r[i]), abs=float(absum[i]))
    return (bool(ok_g.all()), bool(ok_s.all()), float(np.max(rg, initial=0.0)),
            float(np.max(rs, initial=0.0)), first)

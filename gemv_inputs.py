"""Seeded synthetic inputs for the dense GEMV c = B @ a.

This module is shared by the tests, the benchmark and the smoke check. It holds
no GEMV arithmetic: it draws random numbers, casts them to the 16-bit input
dtype and returns raw bit patterns (numpy ``uint16``). The CPU oracle and the
HIP library then read exactly the same bits.

Recipe (the pages print no input data; their GEMV workloads are LLM weight
matrices times an activation vector, TileLang Case Studies, Case B.3 "Shapes
Added"):
  * ``torch.Generator().manual_seed(seed)``, B drawn first, then a;
  * "normal":  B = randn(n, k) / sqrt(k),            a = randn(k);
  * "uniform": B = (2 * rand(n, k) - 1) / sqrt(k),   a = 2 * rand(k) - 1;
  * drawn in float32, then cast to fp16/bf16 by torch (round to nearest even).
"""
import math

import numpy as np
import torch

F16 = 0
BF16 = 1
DTYPE_NAMES = {F16: "f16", BF16: "bf16"}
_TORCH_DTYPE = {F16: torch.float16, BF16: torch.bfloat16}


def torch_dtype(dtype: int) -> torch.dtype:
    return _TORCH_DTYPE[dtype]


def _to_bits(t: torch.Tensor, dtype: int) -> np.ndarray:
    return t.to(_TORCH_DTYPE[dtype]).contiguous().view(torch.int16).numpy().view(np.uint16)


def random_inputs(n: int, k: int, dtype: int, dist: str = "normal", seed: int = 0):
    """Return (B_bits (n, k) uint16, a_bits (k,) uint16)."""
    g = torch.Generator().manual_seed(seed)
    scale = 1.0 / math.sqrt(k) if k > 0 else 1.0
    if dist == "normal":
        B = torch.randn(n, k, generator=g, dtype=torch.float32) * scale
        a = torch.randn(k, generator=g, dtype=torch.float32)
    elif dist == "uniform":
        B = (torch.rand(n, k, generator=g, dtype=torch.float32) * 2 - 1) * scale
        a = torch.rand(k, generator=g, dtype=torch.float32) * 2 - 1
    else:
        raise ValueError("unknown distribution %r" % dist)
    return _to_bits(B, dtype), _to_bits(a, dtype)


def integer_inputs(n: int, k: int, dtype: int, lo: int = -2, hi: int = 2, seed: int = 0):
    """Integer-valued B and a, uniform over [lo, hi] (exactly representable)."""
    g = torch.Generator().manual_seed(seed)
    B = torch.randint(lo, hi + 1, (n, k), generator=g).to(torch.float32)
    a = torch.randint(lo, hi + 1, (k,), generator=g).to(torch.float32)
    return _to_bits(B, dtype), _to_bits(a, dtype)


def values_to_bits(values, dtype: int) -> np.ndarray:
    """Cast float values (already representable, e.g. small integers or
    hand-picked dyadic values) to 16-bit patterns via torch."""
    t = torch.as_tensor(np.asarray(values, dtype=np.float32))
    return _to_bits(t, dtype)


# The workloads: (name, n, k, dtype, distribution).  Shapes are LLM projection
# shapes (TileLang Case Studies, Case B and B.3); the ragged/small-n ones
# exercise the k tails, misaligned rows and the split-k path.
TINY = ("tiny_256x512_f16", 256, 512, F16, "uniform")
PROD_F16 = ("gemv_18432x7168_f16", 18432, 7168, F16, "normal")
PROD_BF16 = ("gemv_7168x16384_bf16", 7168, 16384, BF16, "normal")
SWEEP_SHAPES = [(4096, 4096), (11008, 4096), (4096, 11008), (14336, 4096), (4096, 14336)]
SWEEP = [("sweep_%dx%d_%s" % (n, k, DTYPE_NAMES[d]), n, k, d, "normal")
         for (n, k) in SWEEP_SHAPES for d in (F16, BF16)]
RAGGED = [("ragged_%dx%d_bf16" % (n, k), n, k, BF16, "normal")
          for (n, k) in [(64, 65536), (1000, 7000), (18433, 7169)]]
ALL_WORKLOADS = [TINY, PROD_F16, PROD_BF16] + SWEEP + RAGGED

# Larger production shapes (TileLang Case Studies, Case B.3 "Shapes Added":
# an MLP gate/up projection and an aggregated MoE output) and the small
# square shape of the Case B results table.
LARGE = [("large_%dx%d_%s" % (n, k, DTYPE_NAMES[d]), n, k, d, "normal")
         for (n, k) in [(28672, 8192), (57344, 7168)] for d in (F16, BF16)]
SQUARE = [("square_1024x1024_f16", 1024, 1024, F16, "normal")]
EXTRA_WORKLOADS = LARGE + SQUARE


def find_workload(name):
    for w in ALL_WORKLOADS + EXTRA_WORKLOADS:
        if w[0] == name:
            return w
    return None


def shape_workload(spec):
    """'n,k,f16|bf16' -> an ad-hoc workload tuple (normal distribution)."""
    n, k, d = spec.split(",")
    dt = {"f16": F16, "bf16": BF16}[d]
    return ("shape_%sx%s_%s" % (n, k, d), int(n), int(k), dt, "normal")


def algorithmic_bytes(n: int, k: int, elem_bytes: int = 2) -> int:
    """Bytes a GEMV must move at least once: B, a and c."""
    return elem_bytes * (n * k + k + n)


# ---- one GLA decode step (TileLang Case Studies, Case D; decode shape of
# Case G: batch 1, 32 heads, DK = DV = 128) ----------------------------------
#
# Recipe: q, k ~ N(0,1)/sqrt(DK); v ~ N(0,1); gk = logsigmoid(N(0,1)) (log
# decays, <= 0); S ~ N(0,1) in float32; drawn in that order from one seeded
# generator, q/k/v/gk cast to the 16-bit dtype.

def gla_inputs(bh: int, dk: int, dv: int, dtype: int, seed: int = 0):
    """Return (q, k, v, gk) uint16 patterns and S float32 (bh, dk, dv)."""
    g = torch.Generator().manual_seed(seed)
    s = 1.0 / math.sqrt(dk) if dk > 0 else 1.0
    q = torch.randn(bh, dk, generator=g) * s
    k = torch.randn(bh, dk, generator=g) * s
    v = torch.randn(bh, dv, generator=g)
    gk = torch.nn.functional.logsigmoid(torch.randn(bh, dk, generator=g))
    S = torch.randn(bh, dk, dv, generator=g, dtype=torch.float32)
    return (_to_bits(q, dtype), _to_bits(k, dtype), _to_bits(v, dtype), _to_bits(gk, dtype),
            S.numpy())


GLA_DECODE = ("gla_decode_b1h32_128x128_bf16", 32, 128, 128, BF16)
GLA_BATCHED = ("gla_decode_b64h32_128x128_bf16", 64 * 32, 128, 128, BF16)
GLA_WORKLOADS = [GLA_DECODE, GLA_BATCHED]


def find_gla_workload(name):
    for w in GLA_WORKLOADS:
        if w[0] == name:
            return w
    return None


def gla_step_bytes(bh: int, dk: int, dv: int, elem_bytes: int = 2) -> int:
    """Bytes one GLA decode step must move at least once: the fp32 state read
    and written, q, k, gk (bh x dk) and v, o (bh x dv)."""
    return 8 * bh * dk * dv + elem_bytes * bh * (3 * dk + 2 * dv)

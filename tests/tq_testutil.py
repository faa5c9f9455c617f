"""Shared checks of the GPU parity tests (no GPU work here; imported by the tests).

* ``assert_t_tight``: T = X L1 as the kernels leave it (fp32 accumulation in
  any order, rounded once to bf16) against the fp64 product, within the
  bound that arithmetic fixes: one bf16 ulp of the larger magnitude (the
  final rounding, half an ulp, plus slack for the ulp changing at a binade
  edge) plus gamma_K * sum_k |x_k| |l_k| for the fp32 sum of K products
  (gamma_K = K u / (1 - K u), u = 2^-24, the standard bound on a recursive
  or blocked sum's rounding error).
* ``bf16_values``: fp32 values rounded to the nearest bf16, ties to even
  (the low-rank branch's input when X arrives in fp32).
"""

from __future__ import annotations

import numpy as np


def bf16_values(x):
    """fp32 -> the nearest bf16 value (ties to even), returned as fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (8 significant bits); the smallest normal spacing below 2^-126."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(a)) - 7).astype(np.int64))


def assert_t_tight(t_gpu, x, l1, what=""):
    """t_gpu (n x r, the kernels' bf16 T as fp32/fp64) against X L1 in fp64, within the bound above."""
    xb = bf16_values(x).astype(np.float64)
    l1 = np.asarray(l1, dtype=np.float64)
    k = xb.shape[1]
    t_ref = xb @ l1
    mag = np.abs(xb) @ np.abs(l1)
    u = 2.0 ** -24
    gamma = k * u / (1.0 - k * u)
    t_gpu = np.asarray(t_gpu, dtype=np.float64)
    bound = bf16_ulp(np.maximum(np.abs(t_gpu), np.abs(t_ref))) + gamma * mag
    err = np.abs(t_gpu - t_ref)
    worst = float((err / bound).max()) if err.size else 0.0
    print(f"  {what} T: max |T - T_ref| / bound = {worst:.3f}", flush=True)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (what, len(bad), bad[:5].tolist())

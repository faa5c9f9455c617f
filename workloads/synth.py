"""Seeded input generators.

Every workload draws from one ``numpy.random.SeedSequence`` whose children are
spawned in a fixed order:

    0: activations X          3: low-rank factor L1
    1: outlier-channel picks   4: low-rank factor L2
    2: weight R (or W)         5: signs of the block-Hadamard rotation

Value distributions (second argument of N(.,.) is the standard deviation):

* X ~ N(0, 1), with ``outlier_count`` distinct seeded channels multiplied by
  ``outlier_scale`` (20 for the small case, 30 otherwise; 0.1 % of d rounded
  to the nearest integer), or i.i.d. Student-t with 3 degrees of freedom.
* R (or the full weight W of the two-subspace workload) ~ N(0, 0.02), fp32.
* L1 ~ N(0, 1/sqrt(d)), L2 ~ N(0, 0.02), both rounded to bf16.

X is rounded to bf16 except for the small case, which keeps fp32 values.
Arrays are returned as float32 numpy arrays; bf16 data holds values that are
exactly representable in bf16 (so ``torch.from_numpy(x).bfloat16()`` is
exact).  X is always drawn at the largest token count of a sweep and sliced,
so every token count of a sweep shares its weights and its leading rows.

The two-subspace workload additionally rotates X and W by an orthogonal
U = D . blockdiag(H_128)/sqrt(128) . P (D: seeded +-1 diagonal, H_128: the
Sylvester Hadamard matrix, P: a permutation that moves the ``d_hi`` rotated
coordinates with the largest weighted energy to the end).  That rotation is
part of building the input: the layer receives X' = X U (bf16) and packs
W' = U^T W (fp32).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_STREAMS = 6


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, value recipe and seed."""

    name: str
    title: str
    d: int
    m: int
    r: int
    ns: tuple
    x_kind: str = "normal"  # "normal" (+ outlier channels) or "student_t"
    x_dtype: str = "bf16"  # "f32" or "bf16"
    outlier_count: int = 0
    outlier_scale: float = 1.0
    d_hi: int = 0
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def n(self) -> int:
        return max(self.ns)


def _outliers(d: int) -> int:
    return int(round(0.001 * d))


WORKLOADS = {
    "small": Workload(
        name="small",
        title="small linear 16x512x512 r16 (fp32 X)",
        d=512, m=512, r=16, ns=(16,), x_kind="normal", x_dtype="f32",
        outlier_count=4, outlier_scale=20.0, seed=20260601,
    ),
    "attn_proj": Workload(
        name="attn_proj",
        title="Llama-3-8B attention projection 4096x4096x4096 r32",
        d=4096, m=4096, r=32, ns=(4096,), outlier_count=_outliers(4096),
        outlier_scale=30.0, seed=20260602,
    ),
    "mlp_gate_up": Workload(
        name="mlp_gate_up",
        title="Llama-3-8B MLP gate/up d4096 m14336 r64",
        d=4096, m=14336, r=64, ns=(1, 16, 256, 4096),
        outlier_count=_outliers(4096), outlier_scale=30.0, seed=20260603,
    ),
    "mlp_down": Workload(
        name="mlp_down",
        title="Llama-3-8B MLP down d14336 m4096 r64 (Student-t X)",
        d=14336, m=4096, r=64, ns=(1, 8, 32), x_kind="student_t",
        seed=20260604,
    ),
    "two_subspace": Workload(
        name="two_subspace",
        title="Llama-3-70B MLP two-subspace 8192x8192x28672, 128-dim INT8 subspace",
        d=8192, m=28672, r=0, ns=(8192,), outlier_count=_outliers(8192),
        outlier_scale=30.0, d_hi=128, seed=20260605,
    ),
}


def to_bf16_values(a: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bf16 (ties to even); return float32.

    Uses torch's CPU bfloat16 conversion, a library routine.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _streams(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(_STREAMS)]


def _draw_x(rng_x, rng_o, n, d, x_kind, x_dtype, outlier_count, outlier_scale, outliers=True):
    if x_kind == "normal":
        x = rng_x.standard_normal((n, d), dtype=np.float32)
    elif x_kind == "student_t":
        x = rng_x.standard_t(3.0, size=(n, d)).astype(np.float32)
    else:
        raise ValueError(f"unknown x_kind {x_kind!r}")
    chans = np.zeros(0, dtype=np.int64)
    if x_kind == "normal" and outlier_count > 0:
        chans = np.sort(rng_o.choice(d, size=outlier_count, replace=False))
        if outliers:
            x[:, chans] *= np.float32(outlier_scale)
    if x_dtype == "bf16":
        x = to_bf16_values(x)
    elif x_dtype != "f32":
        raise ValueError(f"unknown x_dtype {x_dtype!r}")
    return x, chans


def _draw_weights(rng_w, rng_l1, rng_l2, d, m, r):
    w = (rng_w.standard_normal((d, m), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    l1 = to_bf16_values(rng_l1.standard_normal((d, r), dtype=np.float32) * np.float32(1.0 / math.sqrt(d)))
    l2 = to_bf16_values(rng_l2.standard_normal((r, m), dtype=np.float32) * np.float32(0.02))
    return w, l1, l2


def draw_custom(n, d, m, r, seed, x_kind="normal", x_dtype="bf16", outlier_count=0,
                outlier_scale=1.0, outliers=True):
    """Draw one linear-layer case of arbitrary shape with the recipe above."""
    s = _streams(seed)
    x, chans = _draw_x(s[0], s[1], n, d, x_kind, x_dtype, outlier_count, outlier_scale, outliers)
    r_w, l1, l2 = _draw_weights(s[2], s[3], s[4], d, m, r)
    return {"X": x, "R": r_w, "L1": l1, "L2": l2, "outlier_channels": chans}


def draw_linear(wl: Workload | str, n: int | None = None, outliers: bool = True):
    """Inputs of a rank-augmented workload, X sliced to the first ``n`` tokens.

    ``outliers=False`` draws the same X without scaling its outlier channels,
    so that the whole code range [-7, 7] is exercised.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if wl.d_hi:
        raise ValueError("use draw_two_subspace for the two-subspace workload")
    case = draw_custom(wl.n, wl.d, wl.m, wl.r, wl.seed, wl.x_kind, wl.x_dtype,
                       wl.outlier_count, wl.outlier_scale, outliers)
    if n is not None:
        if n > wl.n:
            raise ValueError(f"n={n} exceeds the drawn {wl.n} tokens")
        case["X"] = np.ascontiguousarray(case["X"][:n])
    return case


def draw_group_custom(n, d, ms, r, seed, x_kind="normal", x_dtype="bf16", outlier_count=0,
                      outlier_scale=1.0, outliers=True):
    """G layers on one input: X as ``draw_custom(seed)``; layer g's R, L1, L2
    (d x ms[g], d x r, r x ms[g]) from the weight streams of the sequence
    seeded ``seed + 7919 g`` (layer 0: the same weights as ``draw_custom``)."""
    s = _streams(seed)
    x, chans = _draw_x(s[0], s[1], n, d, x_kind, x_dtype, outlier_count, outlier_scale, outliers)
    rs, l1s, l2s = [], [], []
    for g, m in enumerate(ms):
        sg = _streams(seed + 7919 * g)
        r_w, l1, l2 = _draw_weights(sg[2], sg[3], sg[4], d, m, r)
        rs.append(r_w)
        l1s.append(l1)
        l2s.append(l2)
    return {"X": x, "Rs": rs, "L1s": l1s, "L2s": l2s, "outlier_channels": chans}


def draw_group(wl: "Workload | str", n: int | None = None, groups: int = 2, outliers: bool = True):
    """Inputs of ``groups`` layers of a workload's shape sharing its X (gate and
    up of an MLP), X sliced to the first ``n`` tokens."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    case = draw_group_custom(wl.n, wl.d, [wl.m] * groups, wl.r, wl.seed, wl.x_kind, wl.x_dtype,
                             wl.outlier_count, wl.outlier_scale, outliers)
    if n is not None:
        if n > wl.n:
            raise ValueError(f"n={n} exceeds the drawn {wl.n} tokens")
        case["X"] = np.ascontiguousarray(case["X"][:n])
    return case


def _sylvester(k: int) -> np.ndarray:
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < k:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != k:
        raise ValueError("block size must be a power of two")
    return h


def draw_two_subspace_custom(n, d, m, d_hi, seed, block=128, outlier_count=0,
                             outlier_scale=30.0, outliers=True, col_chunk=4096):
    """Rotated inputs of a two-subspace case of arbitrary shape.

    Returns the raw X (bf16 values) and W (fp32), the rotation's pieces
    (``signs``, ``block``, ``perm``) and the layer inputs ``Xrot`` (bf16
    values, n x d) and ``Wrot`` (fp32, d x m); the last ``d_hi`` coordinates of
    the rotated space are the high-precision subspace.
    """
    if d % block:
        raise ValueError("d must be a multiple of the Hadamard block")
    s = _streams(seed)
    x, chans = _draw_x(s[0], s[1], n, d, "normal", "bf16", outlier_count, outlier_scale, outliers)
    w = (s[2].standard_normal((d, m), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    signs = np.where(s[5].integers(0, 2, size=d) == 1, 1.0, -1.0)
    h = _sylvester(block) / math.sqrt(block)
    nb = d // block

    # X . D . blockdiag(H)/sqrt(block), fp64
    xr = (x.astype(np.float64) * signs[None, :]).reshape(n, nb, block) @ h
    xr = xr.reshape(n, d)
    # blockdiag(H)^T/sqrt(block) . D . W, fp64, column chunks to bound memory
    wr = np.empty((d, m), dtype=np.float64)
    for c0 in range(0, m, col_chunk):
        c1 = min(m, c0 + col_chunk)
        blk = (w[:, c0:c1].astype(np.float64) * signs[:, None]).reshape(nb, block, c1 - c0)
        wr[:, c0:c1] = np.matmul(h.T[None], blk).reshape(d, c1 - c0)

    # weighted energy of each rotated coordinate; keep the top d_hi at the end
    x_f2 = float(np.sum(x.astype(np.float64) ** 2))
    w_f2 = float(np.sum(w.astype(np.float64) ** 2))
    score = w_f2 * np.sum(xr * xr, axis=0) + x_f2 * np.sum(wr * wr, axis=1)
    order = np.lexsort((np.arange(d), -score))  # descending score, ties to lower index
    hi = np.sort(order[:d_hi]) if d_hi else np.zeros(0, dtype=np.int64)
    lo_mask = np.ones(d, dtype=bool)
    lo_mask[hi] = False
    perm = np.concatenate([np.nonzero(lo_mask)[0], hi]).astype(np.int64)

    xrot = to_bf16_values(xr[:, perm])
    wrot = wr[perm, :].astype(np.float32)
    del wr
    return {"X": x, "W": w, "signs": signs, "block": block, "perm": perm,
            "hi_index": hi, "Xrot": xrot, "Wrot": wrot, "d_hi": d_hi,
            "outlier_channels": chans}


def draw_two_subspace(wl: Workload | str = "two_subspace", n: int | None = None, outliers=True):
    """Inputs of the two-subspace workload (optionally fewer tokens)."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    case = draw_two_subspace_custom(wl.n, wl.d, wl.m, wl.d_hi, wl.seed,
                                    outlier_count=wl.outlier_count,
                                    outlier_scale=wl.outlier_scale, outliers=outliers)
    if n is not None:
        for k in ("X", "Xrot"):
            case[k] = np.ascontiguousarray(case[k][:n])
    return case

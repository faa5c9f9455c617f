"""Seeded input generators: determinism, shapes, dtypes and value recipes."""

from __future__ import annotations

import numpy as np
import pytest

import oracle.tq_oracle as tqo
from workloads import WORKLOADS, draw_custom, draw_linear, draw_two_subspace_custom, to_bf16_values


def _is_bf16(a):
    return np.all((a.view(np.uint32) & 0xFFFF) == 0)


def test_bf16_rounding_matches_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125: ties to the even 1.0
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)], dtype=np.float32)
    assert to_bf16_values(v).tolist() == [1.0, 1.015625, -1.0]


def test_small_workload_recipe():
    wl = WORKLOADS["small"]
    a = draw_linear(wl)
    b = draw_linear(wl)
    for k in ("X", "R", "L1", "L2"):
        assert np.array_equal(a[k], b[k]), k
    assert a["X"].shape == (16, 512) and a["R"].shape == (512, 512)
    assert a["L1"].shape == (512, 16) and a["L2"].shape == (16, 512)
    assert not _is_bf16(a["X"])  # fp32 activations
    assert _is_bf16(a["L1"]) and _is_bf16(a["L2"])
    assert a["outlier_channels"].size == 4
    ch = a["outlier_channels"]
    plain = np.delete(a["X"], ch, axis=1)
    assert abs(plain.std() - 1.0) < 0.05
    assert a["X"][:, ch].std() > 10  # x20 channels
    assert abs(a["R"].std() - 0.02) < 0.001
    assert abs(a["L1"].std() - 1 / np.sqrt(512)) < 0.005
    # without outliers the same draw is unscaled
    c = draw_linear(wl, outliers=False)
    assert np.array_equal(np.delete(c["X"], ch, axis=1), plain)
    assert c["X"][:, ch].std() < 2


def test_outlier_counts_follow_the_tenth_percent():
    assert WORKLOADS["attn_proj"].outlier_count == 4
    assert WORKLOADS["mlp_gate_up"].outlier_count == 4
    assert WORKLOADS["two_subspace"].outlier_count == 8
    assert WORKLOADS["mlp_down"].x_kind == "student_t"


def test_sweep_slices_share_rows():
    case = draw_custom(64, 256, 96, 8, seed=3, outlier_count=2, outlier_scale=30.0)
    again = draw_custom(64, 256, 96, 8, seed=3, outlier_count=2, outlier_scale=30.0)
    assert np.array_equal(case["X"], again["X"])
    assert _is_bf16(case["X"])
    other = draw_custom(64, 256, 96, 8, seed=4, outlier_count=2, outlier_scale=30.0)
    assert not np.array_equal(case["X"], other["X"])


def test_student_t_heavy_tails():
    case = draw_custom(32, 2048, 16, 4, seed=5, x_kind="student_t")
    x = case["X"]
    assert _is_bf16(x)
    kurt = np.mean(x.astype(np.float64) ** 4) / np.mean(x.astype(np.float64) ** 2) ** 2
    assert kurt > 6  # a Gaussian has 3


def test_two_subspace_inputs_match_the_oracle_rotation():
    n, d, m, dh = 12, 512, 40, 64
    case = draw_two_subspace_custom(n, d, m, dh, seed=11, outlier_count=2)
    u = tqo.block_rotation(case["signs"], case["block"], case["perm"])
    xu, uw = tqo.rotate(case["X"], case["W"], u)
    # the layer inputs are X U rounded to bf16 and U^T W rounded to fp32
    assert _is_bf16(case["Xrot"])
    assert np.all(np.abs(case["Xrot"] - xu) <= 2.0 ** -8 * np.abs(xu) + 1e-30)
    assert np.allclose(case["Wrot"], uw, rtol=2.0 ** -23, atol=1e-12)
    # the high subspace is the last d_hi coordinates and holds the top scores
    assert np.array_equal(case["perm"][d - dh:], case["hi_index"])
    xl, xh, wl, wh = tqo.subspace_split(case["X"], case["W"], u, dh)
    ex = case["X"].astype(np.float64) @ case["W"].astype(np.float64)
    assert np.allclose(xl @ wl + xh @ wh, ex, rtol=1e-10, atol=1e-10)
    # the selected coordinates carry more energy than the rest
    e = np.sum(xu * xu, axis=0)
    assert e[d - dh:].mean() > e[: d - dh].mean()


@pytest.mark.slow
def test_full_size_shapes_gate_up():
    case = draw_linear("mlp_gate_up", n=16)
    assert case["X"].shape == (16, 4096) and case["R"].shape == (4096, 14336)
    full = draw_linear("mlp_gate_up")
    assert np.array_equal(full["X"][:16], case["X"])

"""GPU parity of the two-subspace layer with the rotation applied online (tq_linear_mp_rht) against the CPU oracle.

Bar: the fp32 rotated rows are reproduced bit for bit (the oracle fixes the butterfly order), so both subspaces'
codes and scales are bit-exact; Y within max|Y - Y_ref| <= 1e-2 * max|Y_ref|.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.tq_oracle as tqo  # noqa: E402
import rank_augmented_quantized_amd as tq  # noqa: E402
from workloads import WORKLOADS, draw_two_subspace, draw_two_subspace_custom  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 1e-2
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.load()


def _t(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def _int8_codes(b):
    n, d = b.shape
    v = b.view(np.int8).astype(np.int16).reshape(n, d // 8, 2, 4)
    return np.stack([v[:, :, 0, :], v[:, :, 1, :]], axis=-1).reshape(n, d)


def _run(x, xdt, signs, perm, wrot, d_hi):
    n, d = x.shape
    m = wrot.shape[1]
    dl = d - d_hi
    wlc, swl = tq.tq_pack_weight(_t(np.ascontiguousarray(wrot[:dl])), 4) if dl else (None, None)
    whc, swh = tq.tq_pack_weight(_t(np.ascontiguousarray(wrot[dl:])), 8) if d_hi else (None, None)
    rot = tq.tq_pack_rht(_t(np.asarray(signs, np.float32)), _t(np.asarray(perm, np.int32)))
    ws = torch.zeros(max(1, tq.tq_linear_mp_workspace_bytes(n, d, d_hi)), dtype=torch.uint8, device=DEV)
    xt = _t(x, torch.bfloat16 if xdt == "bf16" else torch.float32)
    y = tq.tq_linear_mp_rht(xt, d_hi, rot, wlc, swl, whc, swh, m, ws=ws)
    torch.cuda.synchronize()
    return y, ws


def _check_codes(ws, n, d, d_hi, ref, rows=None):
    off = tq.tq_linear_mp_workspace_offsets(n, d, d_hi)
    b = ws.cpu().numpy()
    dl = d - d_hi
    rows = np.arange(n) if rows is None else np.asarray(rows)
    if dl:
        sxl = b[off["s_xl"]: off["s_xl"] + 4 * n].view(np.float32)[rows]
        xl = _int8_codes(b[off["x_codes_l"]: off["x_codes_l"] + n * dl].reshape(n, dl))[rows]
        assert np.array_equal(sxl, ref["s_xl"])
        assert np.array_equal(xl, ref["codes_xl"])
    if d_hi:
        sxh = b[off["s_xh"]: off["s_xh"] + 4 * n].view(np.float32)[rows]
        xh = b[off["x_codes_h"]: off["x_codes_h"] + n * d_hi].reshape(n, d_hi).view(np.int8).astype(np.int16)[rows]
        assert np.array_equal(sxh, ref["s_xh"])
        assert np.array_equal(xh, ref["codes_xh"])


def _assert_y(y, ref_y, what):
    yh = y.float().cpu().numpy().astype(np.float64)
    scale = np.abs(ref_y).max()
    err = np.abs(yh - ref_y).max()
    print(f"  {what}: max|Y-Yref|/max|Yref| = {err / max(scale, 1e-300):.3e}", flush=True)
    assert err <= TOL * scale, (what, err, scale)


@pytest.mark.parametrize("n,d,m,dh,xdt", [(40, 512, 96, 128, "bf16"), (130, 1024, 272, 128, "bf16"),
                                          (16, 256, 64, 0, "bf16"), (70, 256, 80, 256, "bf16"),
                                          (9, 8192, 48, 128, "bf16"), (300, 1024, 200, 384, "f32"),
                                          (1, 128, 32, 32, "bf16"), (33, 2048, 64, 1024, "f32")])
def test_linear_mp_rht(n, d, m, dh, xdt):
    """Ragged tails, every chunk count (d = 128 .. 8192), high subspaces of 0 .. d columns, fp32 and bf16 X."""
    print(f"case rht n={n} d={d} m={m} d_hi={dh} {xdt}", flush=True)
    c = draw_two_subspace_custom(n, d, m, dh, seed=5000 + n + d + m, outlier_count=2)
    x = c["X"] if xdt == "bf16" else c["X"] + np.float32(1e-3) * np.random.default_rng(n).standard_normal(
        c["X"].shape).astype(np.float32)
    y, ws = _run(x, xdt, c["signs"], c["perm"], c["Wrot"], dh)
    ref = tqo.tq_linear_mp_rht_ref(x, c["signs"], c["perm"], c["Wrot"], dh)
    _check_codes(ws, n, d, dh, ref)
    _assert_y(y, ref["Y"], f"rht n={n} d={d} dh={dh}")


def test_linear_mp_rht_workload():
    """The 70B MLP shape (8192 x 8192 x 28672, 128-dim 8-bit subspace), sampled rows and columns."""
    w = WORKLOADS["two_subspace"]
    print(f"case rht {w.title}", flush=True)
    c = draw_two_subspace(w)
    y, ws = _run(c["X"], "bf16", c["signs"], c["perm"], c["Wrot"], w.d_hi)
    rng = np.random.default_rng(6)
    rows = np.sort(rng.choice(w.n, 24, replace=False))
    cols = np.sort(rng.choice(w.m, 48, replace=False))
    ref = tqo.tq_linear_mp_rht_ref(c["X"], c["signs"], c["perm"], c["Wrot"], w.d_hi, rows=rows, cols=cols)
    _check_codes(ws, w.n, w.d, w.d_hi, ref, rows=rows)
    _assert_y(y[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)], ref["Y"], "rht workload")

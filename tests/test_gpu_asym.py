"""GPU parity of the two-subspace layer with per-token asymmetric activations against the CPU oracle, through the C ABI.

Bar: weight code sums, per-subspace scales, zero-points and activation codes
bit-exact (stored as u - 8 / u - 128); Y within
max|Y - Y_ref| <= 1e-2 * max|Y_ref| (fp64 oracle).
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
    """int8 code rows in the tile GEMM's order (per 8: the 4 even, then the 4 odd) -> natural order."""
    n, k = b.shape
    v = b.view(np.int8).astype(np.int16).reshape(n, k // 8, 2, 4)
    return np.stack([v[:, :, 0, :], v[:, :, 1, :]], axis=-1).reshape(n, k)


def _run(xrot, wrot, d_hi, x_dtype=torch.bfloat16, y_dtype=torch.bfloat16):
    n, d = xrot.shape
    m = wrot.shape[1]
    dl = d - d_hi
    wl = tq.tq_pack_weight(_t(np.ascontiguousarray(wrot[:dl])), 4) if dl else (None, None)
    wh = tq.tq_pack_weight(_t(np.ascontiguousarray(wrot[dl:])), 8) if d_hi else (None, None)
    csl = tq.tq_weight_colsum(wl[0], dl, 4) if dl else None
    csh = tq.tq_weight_colsum(wh[0], d_hi, 8) if d_hi else None
    ws = torch.empty(max(1, tq.tq_linear_mp_asym_workspace_bytes(n, d, d_hi)), dtype=torch.uint8, device=DEV)
    xt = _t(xrot, x_dtype)
    y = tq.tq_linear_mp_asym(xt, d_hi, wl[0], wl[1], csl, wh[0], wh[1], csh, m, y_dtype=y_dtype, ws=ws)
    torch.cuda.synchronize()
    # the same call through tq_linear_mp_asym_debug: the kernel's int32 sums of the stored codes of both subspaces
    acc_l = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV)
    acc_h = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV) if d_hi else None
    ws2 = torch.empty_like(ws)
    y2 = tq.tq_linear_mp_asym(xt, d_hi, wl[0], wl[1], csl, wh[0], wh[1], csh, m, y_dtype=y_dtype, ws=ws2,
                              acc_l=acc_l, acc_h=acc_h)
    torch.cuda.synchronize()
    assert torch.equal(y2, y), "the accumulator-export call changed Y"
    _run.acc = (acc_l.cpu().numpy().astype(np.int64),
                acc_h.cpu().numpy().astype(np.int64) if d_hi else np.zeros((n, m), np.int64))
    return y, ws, csl, csh


def _ws_parts(ws, n, d, d_hi):
    off = tq.tq_linear_mp_asym_workspace_offsets(n, d, d_hi)
    dl = d - d_hi
    b = ws.cpu().numpy()
    f = {k: b[off[k]: off[k] + 4 * n].view(np.float32) for k in ("s_xl", "s_xh", "z_xl", "z_xh")}
    ul = _int8_codes(b[off["x_codes_l"]: off["x_codes_l"] + n * dl].reshape(n, dl)) + 8 if dl else None
    uh = b[off["x_codes_h"]: off["x_codes_h"] + n * d_hi].reshape(n, d_hi).view(np.int8).astype(np.int16) + 128 \
        if d_hi else None
    return f, ul, uh


def _check(xrot, wrot, d_hi, y, ws, csl, csh, rows=None, cols=None):
    n, d = xrot.shape
    dl = d - d_hi
    ref = tqo.tq_linear_mp_asym_ref(xrot, wrot, d_hi, rows=rows, cols=cols)
    f, ul, uh = _ws_parts(ws, n, d, d_hi)
    r = slice(None) if rows is None else rows
    if dl:
        assert np.array_equal(f["s_xl"][r], ref["s_xl"]) and np.array_equal(f["z_xl"][r], ref["z_xl"])
        assert np.array_equal(ul[r], ref["codes_xl"])
        if cols is None:
            assert np.array_equal(csl.cpu().numpy(), ref["colsum_l"])
    if d_hi:
        assert np.array_equal(f["s_xh"][r], ref["s_xh"]) and np.array_equal(f["z_xh"][r], ref["z_xh"])
        assert np.array_equal(uh[r], ref["codes_xh"])
        if cols is None:
            assert np.array_equal(csh.cpu().numpy(), ref["colsum_h"])
    # sums of the stored codes u - 2^(N-1): U C_w^T - 2^(N-1) colsum of each subspace, exactly
    acc_l, acc_h = _run.acc
    if rows is not None:
        acc_l, acc_h = acc_l[np.ix_(rows, cols)], acc_h[np.ix_(rows, cols)]
    if dl:
        assert np.array_equal(acc_l, ref["acc_l"] - 8 * ref["colsum_l"][None, :])
    if d_hi:
        assert np.array_equal(acc_h, ref["acc_h"] - 128 * ref["colsum_h"][None, :])
    yg = y.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        yg = yg[np.ix_(rows, cols)]
    err = np.abs(yg - ref["Y"]).max()
    scale = np.abs(ref["Y"]).max()
    print(f"  max|Y-Yref|/max|Yref| = {err / scale:.3e}", flush=True)
    assert err <= TOL * scale


@pytest.mark.parametrize("n,d,m,dh", [(40, 512, 96, 64), (130, 1024, 272, 128), (16, 256, 64, 0),
                                      (70, 256, 80, 256), (9, 8192, 48, 128), (300, 1024, 200, 384),
                                      (1, 128, 32, 32), (40, 560, 96, 48), (33, 608, 64, 96),
                                      (512, 1024, 2048, 128)])
def test_linear_mp_asym(n, d, m, dh):
    print(f"case n={n} d={d} m={m} d_hi={dh}", flush=True)
    block = 128 if d % 128 == 0 else 16
    c = draw_two_subspace_custom(n, d, m, dh, seed=900 + n + d + dh, block=block, outlier_count=2)
    y, ws, csl, csh = _run(c["Xrot"], c["Wrot"], dh)
    _check(c["Xrot"], c["Wrot"], dh, y, ws, csl, csh)


def test_linear_mp_asym_fp32_x_and_shifted_rows():
    """fp32 X, fp32 Y, rows shifted away from zero (all-positive and all-negative tokens) and a constant row."""
    n, d, m, dh = 24, 512, 80, 128
    c = draw_two_subspace_custom(n, d, m, dh, seed=97)
    x = c["Xrot"].astype(np.float32).copy()
    x[::3] += 4.0
    x[1::3] -= 7.5
    x[5] = np.float32(0.625)
    y, ws, csl, csh = _run(x, c["Wrot"], dh, torch.float32, torch.float32)
    _check(x, c["Wrot"], dh, y, ws, csl, csh)


def test_linear_mp_asym_workload_sampled():
    """The Llama-2-70B two-subspace shape (8192 tokens, d 8192, m 28672), sampled tokens and channels."""
    w = WORKLOADS["two_subspace"]
    c = draw_two_subspace(w)
    xrot, wrot = c["Xrot"], c["Wrot"]
    d_hi = w.d_hi
    n, d = xrot.shape
    y, ws, csl, csh = _run(xrot, wrot, d_hi)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(n, 24, replace=False))
    cols = np.sort(rng.choice(wrot.shape[1], 48, replace=False))
    _check(xrot, wrot, d_hi, y, ws, csl, csh, rows=rows, cols=cols)

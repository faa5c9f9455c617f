"""GPU parity of the two-subspace layer at 6/3 bits (CoQuant's other bit pair) against the CPU oracle, through the C ABI.

Bar: weight codes and scales, activation codes and scales of both subspaces
bit-exact; Y within max|Y - Y_ref| <= 1e-2 * max|Y_ref| of the fp64 oracle.
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


def _run(xrot, wrot, d_hi, x_dtype=torch.bfloat16):
    n, d = xrot.shape
    m = wrot.shape[1]
    dl = d - d_hi
    wl = tq.tq_pack_weight(_t(np.ascontiguousarray(wrot[:dl])), 3) if dl else (None, None)
    wh = tq.tq_pack_weight(_t(np.ascontiguousarray(wrot[dl:])), 6) if d_hi else (None, None)
    ws = torch.empty(max(1, tq.tq_linear_mp_workspace_bytes(n, d, d_hi)), dtype=torch.uint8, device=DEV)
    xt = _t(xrot, x_dtype)
    y = tq.tq_linear_mp(xt, d_hi, wl[0], wl[1], wh[0], wh[1], m, ws=ws, bits=(3, 6))
    torch.cuda.synchronize()
    # the same call through tq_linear_mp_bits_debug: the kernel's int32 sums of both subspaces
    acc_l = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV)
    acc_h = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV) if d_hi else None
    y2 = tq.tq_linear_mp(xt, d_hi, wl[0], wl[1], wh[0], wh[1], m, ws=torch.empty_like(ws), bits=(3, 6),
                         acc_l=acc_l, acc_h=acc_h)
    torch.cuda.synchronize()
    assert torch.equal(y2, y), "the accumulator-export call changed Y"
    _run.acc = (acc_l.cpu().numpy().astype(np.int64),
                acc_h.cpu().numpy().astype(np.int64) if d_hi else np.zeros((n, m), np.int64))
    return y, ws, wl, wh


def _check(xrot, wrot, d_hi, y, ws, wl, wh, rows=None, cols=None):
    n, d = xrot.shape
    dl = d - d_hi
    ref = tqo.tq_linear_mp_ref(xrot, wrot, d_hi, rows=rows, cols=cols, bits_lo=3, bits_hi=6)
    off = tq.tq_linear_mp_workspace_offsets(n, d, d_hi)
    b = ws.cpu().numpy()
    r = slice(None) if rows is None else rows
    if dl:
        assert np.array_equal(b[off["s_xl"]: off["s_xl"] + 4 * n].view(np.float32)[r], ref["s_xl"])
        xl = _int8_codes(b[off["x_codes_l"]: off["x_codes_l"] + n * dl].reshape(n, dl))
        assert np.array_equal(xl[r], ref["codes_xl"])
        if cols is None:
            assert np.array_equal(tqo.unpack_int4(wl[0].cpu().numpy()), ref["codes_wl"])
            assert np.array_equal(wl[1].cpu().numpy(), ref["s_wl"])
    if d_hi:
        assert np.array_equal(b[off["s_xh"]: off["s_xh"] + 4 * n].view(np.float32)[r], ref["s_xh"])
        xh = b[off["x_codes_h"]: off["x_codes_h"] + n * d_hi].reshape(n, d_hi).view(np.int8).astype(np.int16)
        assert np.array_equal(xh[r], ref["codes_xh"])
        if cols is None:
            assert np.array_equal(wh[0].cpu().numpy().view(np.int8).astype(np.int16), ref["codes_wh"])
            assert np.array_equal(wh[1].cpu().numpy(), ref["s_wh"])
    acc_l, acc_h = _run.acc
    if rows is not None:
        acc_l, acc_h = acc_l[np.ix_(rows, cols)], acc_h[np.ix_(rows, cols)]
    assert np.array_equal(acc_l, ref["acc_l"]) and np.array_equal(acc_h, ref["acc_h"])
    yg = y.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        yg = yg[np.ix_(rows, cols)]
    err = np.abs(yg - ref["Y"]).max()
    scale = np.abs(ref["Y"]).max()
    print(f"  max|Y-Yref|/max|Yref| = {err / scale:.3e}", flush=True)
    assert err <= TOL * scale


@pytest.mark.parametrize("n,d,m,dh", [(40, 512, 96, 64), (130, 1024, 272, 128), (16, 256, 64, 0),
                                      (70, 256, 80, 256), (9, 8192, 48, 128), (300, 1024, 200, 384),
                                      (1, 128, 32, 32), (40, 560, 96, 48), (512, 1024, 2048, 128)])
def test_linear_mp_6_3(n, d, m, dh):
    print(f"case n={n} d={d} m={m} d_hi={dh}", flush=True)
    block = 128 if d % 128 == 0 else 16
    c = draw_two_subspace_custom(n, d, m, dh, seed=700 + n + d + dh, block=block, outlier_count=2)
    y, ws, wl, wh = _run(c["Xrot"], c["Wrot"], dh)
    _check(c["Xrot"], c["Wrot"], dh, y, ws, wl, wh)


def test_linear_mp_6_3_fp32_x_plain():
    """fp32 X without outlier channels (codes over the whole 3- and 6-bit ranges)."""
    n, d, m, dh = 33, 512, 96, 64
    c = draw_two_subspace_custom(n, d, m, dh, seed=71, outliers=False)
    x = c["Xrot"].astype(np.float32)
    y, ws, wl, wh = _run(x, c["Wrot"], dh, torch.float32)
    _check(x, c["Wrot"], dh, y, ws, wl, wh)


def test_linear_mp_6_3_workload_sampled():
    """The Llama-2-70B two-subspace shape (8192 tokens, d 8192, m 28672) at 6/3 bits, sampled."""
    w = WORKLOADS["two_subspace"]
    c = draw_two_subspace(w)
    y, ws, wl, wh = _run(c["Xrot"], c["Wrot"], w.d_hi)
    rng = np.random.default_rng(6)
    rows = np.sort(rng.choice(w.n, 24, replace=False))
    cols = np.sort(rng.choice(w.m, 48, replace=False))
    _check(c["Xrot"], c["Wrot"], w.d_hi, y, ws, wl, wh, rows=rows, cols=cols)

"""GPU parity of the fully quantised low-rank branch against the CPU oracle, through the C ABI.

Layer: Y = s_x s_w (C_x C_w^T) + (s_x s_t) s_v (C_t C_v^T), C_t / s_t the
per-token 4-bit re-quantisation of t = fl32(C_x C_u^T) * s_u.  Bar: packed
codes and scales of U and V, activation codes, s_x, the first stage's codes
and s_t bit-exact; the int32 sums of the residual product and of the second
stage, exported by the kernels that produce Y (tq_linear_qlr_debug, whose Y
must equal the plain call's bit for bit), bit-exact; Y within
max|Y - Y_ref| <= 1e-2 * max|Y_ref| (fp64 oracle).
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.tq_oracle as tqo  # noqa: E402
import rank_augmented_quantized_amd as tq  # noqa: E402
from workloads import draw_custom, draw_linear  # noqa: E402

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


def _r_pad(r):
    p = 32
    while p < r:
        p *= 2
    return p


def _int8_codes(b):
    """int8 code rows in the tile GEMM's order (per 8: the 4 even, then the 4 odd) -> natural order."""
    n, k = b.shape
    v = b.view(np.int8).astype(np.int16).reshape(n, k // 8, 2, 4)
    return np.stack([v[:, :, 0, :], v[:, :, 1, :]], axis=-1).reshape(n, k)


def _pack_parts(buf, d, m, r):
    """U^T codes, s_u, V^T codes, s_v of a tq_pack_lowrank_q buffer (layout of include/tq.h)."""
    rp = _r_pad(r)

    def al(v):
        return (v + 255) & ~255

    b = buf.cpu().numpy()
    o_su = al(rp * d // 2)
    o_vc = al(o_su + 4 * rp)
    o_sv = al(o_vc + m * rp // 2)
    uc = tqo.unpack_int4(b[:rp * d // 2].reshape(rp, d // 2))
    su = b[o_su:o_su + 4 * rp].view(np.float32)
    vc = tqo.unpack_int4(b[o_vc:o_vc + m * rp // 2].reshape(m, rp // 2))
    sv = b[o_sv:o_sv + 4 * m].view(np.float32)
    return uc, su, vc, sv


def _run(x, xdt, r_w, u, v, y_dtype=torch.bfloat16):
    n, d = x.shape
    m, rk = r_w.shape[1], u.shape[1]
    wc, sw = tq.tq_pack_weight(_t(r_w), 4)
    lq = tq.tq_pack_lowrank_q(_t(u), _t(v))
    ws = torch.zeros(max(1, tq.tq_linear_qlr_workspace_bytes(n, d, rk)), dtype=torch.uint8, device=DEV)
    xt = _t(x, torch.bfloat16 if xdt == "bf16" else torch.float32)
    y = tq.tq_linear_qlr(xt, wc, sw, lq, m, rk, y_dtype=y_dtype, ws=ws)
    torch.cuda.synchronize()
    return y, ws, lq


def _acc(x, xdt, r_w, u, v, y):
    """The same layer through tq_linear_qlr_debug: (residual sums, second-stage sums), int64 n x m."""
    n, d = x.shape
    m, rk = r_w.shape[1], u.shape[1]
    wc, sw = tq.tq_pack_weight(_t(r_w), 4)
    lq = tq.tq_pack_lowrank_q(_t(u), _t(v))
    ws = torch.zeros(max(1, tq.tq_linear_qlr_workspace_bytes(n, d, rk)), dtype=torch.uint8, device=DEV)
    acc = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV)
    acc2 = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV)
    y2 = torch.empty_like(y)
    tq.tq_linear_qlr(_t(x, torch.bfloat16 if xdt == "bf16" else torch.float32), wc, sw, lq, m, rk, Y=y2, ws=ws,
                     acc=acc, acc2=acc2)
    torch.cuda.synchronize()
    assert torch.equal(y2, y), "the accumulator-export call changed Y"
    return acc.cpu().numpy().astype(np.int64), acc2.cpu().numpy().astype(np.int64)


def _ws_parts(ws, n, d, rk):
    off = tq.tq_linear_qlr_workspace_offsets(n, d, rk)
    rp = _r_pad(rk)
    b = ws.cpu().numpy()
    sx = b[off["s_x"]: off["s_x"] + 4 * n].view(np.float32)
    if n <= 32:  # few tokens: nibble-packed codes for the small-n GEMM
        xc = tqo.unpack_int4(b[off["x_codes"]: off["x_codes"] + n * d // 2].reshape(n, d // 2))
    else:
        xc = _int8_codes(b[off["x_codes"]: off["x_codes"] + n * d].reshape(n, d))
    st = b[off["s_t"]: off["s_t"] + 4 * n].view(np.float32)
    tc = _int8_codes(b[off["t_codes"]: off["t_codes"] + n * rp].reshape(n, rp))
    return sx, xc, st, tc


CASES = [
    # (name, n, d, m, r, x_kind, x_dtype, outliers)
    ("n1_r32", 1, 512, 256, 32, "normal", "bf16", 2),
    ("n7_r8_ragged_m", 7, 1024, 200, 8, "normal", "f32", 2),
    ("n40_r32_d544_ragged_k", 40, 544, 272, 32, "normal", "bf16", 2),
    ("n300_r64_student_t", 300, 1024, 512, 64, "student_t", "bf16", 0),
    ("n257_r100_rpad128", 257, 2048, 384, 100, "normal", "bf16", 2),
    ("n33_r256", 33, 512, 256, 256, "normal", "f32", 0),
    ("n1030_r32_d4096", 1030, 4096, 1024, 32, "normal", "bf16", 4),
    ("n64_r16_no_outliers", 64, 768, 256, 16, "normal", "bf16", 0),
    ("n70_r32_d5120_two_launch", 70, 5120, 256, 32, "normal", "bf16", 2),
    ("n5_r64_d14336_two_launch", 5, 14336, 128, 64, "student_t", "f32", 0),
    ("n32_r32_small_n", 32, 2048, 520, 32, "normal", "bf16", 2),
    ("n17_r256_small_n_two_launch", 17, 1024, 272, 256, "normal", "bf16", 0),
    ("n2_r64_d4096", 2, 4096, 1024, 64, "normal", "bf16", 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_linear_qlr(case):
    name, n, d, m, rk, kind, xdt, nout = case
    print(f"case {name}", flush=True)
    c = draw_custom(n, d, m, rk, seed=5000 + n + d + rk, x_kind=kind, x_dtype=xdt, outlier_count=nout,
                    outlier_scale=30.0)
    u, v = c["L1"], c["L2"]
    y, ws, lq = _run(c["X"], xdt, c["R"], u, v)
    ref = tqo.tq_linear_qlr_ref(c["X"], c["R"], u, v)
    # packed factors
    uc, su, vc, sv = _pack_parts(lq, d, m, rk)
    assert np.array_equal(uc[:rk], ref["codes_u"]) and not uc[rk:].any()
    assert np.array_equal(su[:rk], ref["s_u"]) and not su[rk:].any()
    assert np.array_equal(vc[:, :rk], ref["codes_v"]) and not vc[:, rk:].any()
    assert np.array_equal(sv, ref["s_v"])
    # activations and the re-quantised first stage
    sx, xc, st, tc = _ws_parts(ws, n, d, rk)
    assert np.array_equal(sx, ref["s_x"])
    assert np.array_equal(xc, ref["codes_x"])
    assert np.array_equal(st, ref["s_t"])
    assert np.array_equal(tc[:, :rk], ref["codes_t"]) and not tc[:, rk:].any()
    acc, acc2 = _acc(c["X"], xdt, c["R"], u, v, y)
    assert np.array_equal(acc, ref["acc"])
    assert np.array_equal(acc2, ref["acc2"])
    err = np.abs(y.float().cpu().numpy().astype(np.float64) - ref["Y"]).max()
    scale = np.abs(ref["Y"]).max()
    print(f"  max|Y-Yref|/max|Yref| = {err / scale:.3e}", flush=True)
    assert err <= TOL * scale


def test_linear_qlr_fp32_output_and_zero_v():
    """fp32 Y; V = 0 gives the plain W4A4 layer of tq_linear with r = 0, bit for bit."""
    n, d, m, rk = 70, 512, 256, 32
    c = draw_custom(n, d, m, rk, seed=77)
    y, *_ = _run(c["X"], "bf16", c["R"], c["L1"], np.zeros_like(c["L2"]), torch.float32)
    wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
    y0 = tq.tq_linear(_t(c["X"], torch.bfloat16), wc, sw, None, m, 0, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)


def test_linear_qlr_attn_proj_sampled():
    """Llama-3-8B attention projection (n = d = m = 4096, r = 32) in the launch configuration the
    benchmark times, checked on sampled tokens and channels (every step is row- or column-local)."""
    c = draw_linear("attn_proj")
    x, r_w, u, v = c["X"], c["R"], c["L1"], c["L2"]
    n, d = x.shape
    m, rk = r_w.shape[1], u.shape[1]
    y, ws, _ = _run(x, "bf16", r_w, u, v)
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(n, 48, replace=False))
    cols = np.sort(rng.choice(m, 64, replace=False))
    ref = tqo.tq_linear_qlr_ref(x, r_w, u, v, rows=rows, cols=cols)
    sx, xc, st, tc = _ws_parts(ws, n, d, rk)
    assert np.array_equal(sx[rows], ref["s_x"]) and np.array_equal(xc[rows], ref["codes_x"])
    assert np.array_equal(st[rows], ref["s_t"]) and np.array_equal(tc[rows, :rk], ref["codes_t"])
    yg = y.float().cpu().numpy().astype(np.float64)[np.ix_(rows, cols)]
    err = np.abs(yg - ref["Y"]).max()
    scale = np.abs(ref["Y"]).max()
    print(f"  sampled max|Y-Yref|/max|Yref| = {err / scale:.3e}", flush=True)
    assert err <= TOL * scale


def test_linear_qlr_graph_replay_matches_eager():
    """The layer's launches captured in a HIP graph and replayed give the eager output on every replay."""
    n, d, m, rk = 300, 1024, 512, 32
    c = draw_custom(n, d, m, rk, seed=79)
    wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
    lq = tq.tq_pack_lowrank_q(_t(c["L1"]), _t(c["L2"]))
    x = _t(c["X"], torch.bfloat16)
    ws = torch.zeros(tq.tq_linear_qlr_workspace_bytes(n, d, rk), dtype=torch.uint8, device=DEV)
    y = torch.empty((n, m), dtype=torch.bfloat16, device=DEV)
    tq.tq_linear_qlr(x, wc, sw, lq, m, rk, Y=y, ws=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tq.tq_linear_qlr(x, wc, sw, lq, m, rk, Y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tq.tq_linear_qlr(x, wc, sw, lq, m, rk, Y=y, ws=ws)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)

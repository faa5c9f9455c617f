"""GPU parity of the rank-augmented layer with per-token asymmetric activations against the CPU oracle, through the C ABI.

Bar: s_x, z_x, the activation codes (stored as u - 8) and the weight code
sums bit-exact; T within 2e-2 of each row's max (bf16); Y within
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


def _int8_codes(b):
    """int8 code rows in the tile GEMM's order (per 8: the 4 even, then the 4 odd) -> natural order."""
    n, k = b.shape
    v = b.view(np.int8).astype(np.int16).reshape(n, k // 8, 2, 4)
    return np.stack([v[:, :, 0, :], v[:, :, 1, :]], axis=-1).reshape(n, k)


def _r_pad(r):
    p = 32
    while p < r:
        p *= 2
    return p if r else 0


def _run(x, xdt, r_w, l1, l2):
    n, d = x.shape
    m = r_w.shape[1]
    rk = 0 if l1 is None else l1.shape[1]
    wc, sw = tq.tq_pack_weight(_t(r_w), 4)
    cs = tq.tq_weight_colsum(wc, d, 4)
    lr = tq.tq_pack_lowrank(_t(l1, torch.bfloat16), _t(l2, torch.bfloat16)) if rk else None
    ws = torch.zeros(tq.load().tq_linear_asym_workspace_bytes(n, d, m, rk), dtype=torch.uint8, device=DEV)
    xt = _t(x, torch.bfloat16 if xdt == "bf16" else torch.float32)
    y = tq.tq_linear_asym(xt, wc, sw, cs, lr, m, rk, ws=ws)
    torch.cuda.synchronize()
    # the same call through tq_linear_asym_debug: the kernels' int32 sums of the stored codes u - 8
    acc = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV)
    y2 = torch.empty_like(y)
    ws2 = torch.zeros(tq.load().tq_linear_asym_workspace_bytes(n, d, m, rk), dtype=torch.uint8, device=DEV)
    tq.tq_linear_asym(xt, wc, sw, cs, lr, m, rk, Y=y2, ws=ws2, acc=acc)
    torch.cuda.synchronize()
    assert torch.equal(y2, y), "the accumulator-export call changed Y"
    _run.acc = acc.cpu().numpy().astype(np.int64)
    return y, ws, cs


def _check(x, r_w, l1, l2, y, ws, cs, rows=None, cols=None):
    n, d = x.shape
    m = r_w.shape[1]
    rk = 0 if l1 is None else l1.shape[1]
    ref = tqo.tq_linear_asym_ref(x, r_w, l1, l2, rows=rows, cols=cols)
    off = tq.tq_linear_asym_workspace_offsets(n, d, m, rk)
    b = ws.cpu().numpy()
    r = slice(None) if rows is None else rows
    assert np.array_equal(b[off["s_x"]: off["s_x"] + 4 * n].view(np.float32)[r], ref["s_x"])
    assert np.array_equal(b[off["z_x"]: off["z_x"] + 4 * n].view(np.float32)[r], ref["z_x"])
    if n <= 32:  # few tokens: nibble-packed codes for the small-n GEMM
        codes = tqo.unpack_int4(b[off["x_codes"]: off["x_codes"] + n * d // 2].reshape(n, d // 2)) + 8
    else:
        codes = _int8_codes(b[off["x_codes"]: off["x_codes"] + n * d].reshape(n, d)) + 8
    assert np.array_equal(codes[r], ref["codes_x"])
    if cols is None:
        assert np.array_equal(cs.cpu().numpy(), ref["colsum"])
    # the kernels' sums over the stored codes u - 8: U C_w^T - 8 colsum, exactly
    acc = _run.acc if rows is None else _run.acc[np.ix_(rows, cols)]
    assert np.array_equal(acc, ref["acc"] - 8 * ref["colsum"][None, :])
    if rk:
        rp = _r_pad(rk)
        t = ws[off["T"]: off["T"] + n * rp * 2].view(torch.bfloat16).view(n, rp).float().cpu().numpy()[r, :rk]
        scale = np.abs(ref["T"]).max(axis=1, keepdims=True) + 1e-30
        assert (np.abs(t - ref["T"]) / scale).max() <= 2e-2
    yg = y.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        yg = yg[np.ix_(rows, cols)]
    err = np.abs(yg - ref["Y"]).max()
    scale = np.abs(ref["Y"]).max()
    print(f"  max|Y-Yref|/max|Yref| = {err / scale:.3e}", flush=True)
    assert err <= TOL * scale


CASES = [
    # (name, n, d, m, r, x_kind, x_dtype, outliers)
    ("n1_r32", 1, 512, 256, 32, "normal", "bf16", 2),
    ("n7_r0_ragged_m", 7, 1024, 200, 0, "normal", "f32", 2),
    ("n40_r16_d544", 40, 544, 272, 16, "normal", "bf16", 2),
    ("n300_r64_student_t", 300, 1024, 512, 64, "student_t", "bf16", 0),
    ("n1030_r32_fused", 1030, 2048, 384, 32, "normal", "bf16", 4),
    ("n1100_r0_fused_f32", 1100, 512, 256, 0, "normal", "f32", 0),
    ("n33_r64_d14336_streamed", 33, 14336, 256, 64, "student_t", "bf16", 0),
    ("n64_r32_d8192", 64, 8192, 128, 32, "normal", "f32", 2),
    ("n2_r64_small_n", 2, 4096, 1024, 64, "normal", "bf16", 2),
    ("n32_r32_small_n", 32, 2048, 520, 32, "normal", "bf16", 0),
    ("n16_r0_small_n_f32", 16, 1024, 256, 0, "normal", "f32", 2),
    ("n3_r32_d16384_max_small_n", 3, 16384, 256, 32, "student_t", "bf16", 0),
    ("n40_r16_d16384_max", 40, 16384, 128, 16, "normal", "f32", 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_linear_asym(case):
    name, n, d, m, rk, kind, xdt, nout = case
    print(f"case {name}", flush=True)
    c = draw_custom(n, d, m, max(rk, 1), seed=6000 + n + d + rk, x_kind=kind, x_dtype=xdt, outlier_count=nout,
                    outlier_scale=30.0)
    l1 = c["L1"] if rk else None
    l2 = c["L2"] if rk else None
    x = c["X"]
    if name.startswith("n1100"):
        x = (x + np.float32(3.0)).astype(np.float32)  # all-positive rows: z far from 0
    y, ws, cs = _run(x, xdt, c["R"], l1, l2)
    _check(x, c["R"], l1, l2, y, ws, cs)


def test_linear_asym_attn_proj_sampled():
    """Llama-3-8B attention projection (4096^3, r 32) with asymmetric activations, sampled."""
    c = draw_linear("attn_proj")
    y, ws, cs = _run(c["X"], "bf16", c["R"], c["L1"], c["L2"])
    rng = np.random.default_rng(12)
    rows = np.sort(rng.choice(4096, 48, replace=False))
    cols = np.sort(rng.choice(4096, 64, replace=False))
    _check(c["X"], c["R"], c["L1"], c["L2"], y, ws, cs, rows=rows, cols=cols)


def test_linear_asym_graph_replay_matches_eager():
    """The asymmetric layer (quantiser, T blocks with their cross-block counters, GEMM) captured in a HIP graph
    and replayed gives the eager output on every replay."""
    n, d, m, rk = 300, 2048, 512, 32
    c = draw_custom(n, d, m, rk, seed=81)
    wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
    cs = tq.tq_weight_colsum(wc, d, 4)
    lr = tq.tq_pack_lowrank(_t(c["L1"], torch.bfloat16), _t(c["L2"], torch.bfloat16))
    x = _t(c["X"], torch.bfloat16)
    ws = torch.zeros(tq.load().tq_linear_asym_workspace_bytes(n, d, m, rk), dtype=torch.uint8, device=DEV)
    y = torch.empty((n, m), dtype=torch.bfloat16, device=DEV)
    tq.tq_linear_asym(x, wc, sw, cs, lr, m, rk, Y=y, ws=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tq.tq_linear_asym(x, wc, sw, cs, lr, m, rk, Y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tq.tq_linear_asym(x, wc, sw, cs, lr, m, rk, Y=y, ws=ws)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)


@pytest.mark.parametrize("n,d,m,rk,launches", [(16, 4096, 300, 64, {"small_fused_asym"}),
                                               (5, 14336, 80, 64, {"small_fused_asym"}),
                                               (24, 2048, 200, 32, {"prologue_asym", "gemm_small_n_asym"})])
def test_linear_asym_few_token_launches(n, d, m, rk, launches):
    """Up to 16 tokens the asymmetric layer runs in one launch (the producer blocks quantise with a zero-point),
    17 .. 32 in two; both give codes, scales, zero-points and accumulators bit-exact and Y within the tolerance,
    and the hand-off words are zero again after each call."""
    print(f"case n={n} d={d} m={m} r={rk}", flush=True)
    c = draw_custom(n, d, m, rk, seed=7100 + n, outlier_count=2, outlier_scale=30.0)
    wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
    cs = tq.tq_weight_colsum(wc, d, 4)
    lr = tq.tq_pack_lowrank(_t(c["L1"], torch.bfloat16), _t(c["L2"], torch.bfloat16))
    ws = torch.zeros(tq.load().tq_linear_asym_workspace_bytes(n, d, m, rk), dtype=torch.uint8, device=DEV)
    xt = _t(c["X"], torch.bfloat16)
    tq.tq_profile_reset()
    tq.tq_profile_enable(True)
    y = tq.tq_linear_asym(xt, wc, sw, cs, lr, m, rk, ws=ws)
    torch.cuda.synchronize()
    tq.tq_profile_enable(False)
    names = set(tq.tq_profile_read())
    tq.tq_profile_reset()
    assert names == launches, names
    assert not ws[:4096].view(torch.int32).cpu().numpy().any()
    y_again = tq.tq_linear_asym(xt, wc, sw, cs, lr, m, rk, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y_again, y)
    y_run, ws_run, cs_run = _run(c["X"], "bf16", c["R"], c["L1"], c["L2"])
    assert torch.equal(y_run, y)
    _check(c["X"], c["R"], c["L1"], c["L2"], y_run, ws_run, cs_run)

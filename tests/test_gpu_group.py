"""GPU parity of grouped layers (several weights on one input) against the CPU oracle, through the C ABI.

Bar as for the single layer: activation codes, scales and every layer's int32
accumulators bit-exact; each layer's block of Y within
max|Y - Y_ref| <= 1e-2 * max|Y_ref| of that layer (fp64 oracle).
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.tq_oracle as tqo  # noqa: E402
import rank_augmented_quantized_amd as tq  # noqa: E402
from workloads import draw_group_custom  # noqa: E402

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
    return p if r else 0


def _tcols(G, r):
    return _r_pad(r) if G == 1 else _r_pad(G * _r_pad(r))


def _int8_codes(b):
    """The tile GEMM's int8 activation codes: per 8 k, the 4 even-k codes, then the 4 odd-k codes."""
    n, d = b.shape
    v = b.view(np.int8).astype(np.int16).reshape(n, d // 8, 2, 4)
    return np.stack([v[:, :, 0, :], v[:, :, 1, :]], axis=-1).reshape(n, d)


def _run_group(x, xdt, rs, l1s, l2s, y_dtype=torch.bfloat16):
    n, d = x.shape
    ms = [r.shape[1] for r in rs]
    rk = 0 if l1s is None else l1s[0].shape[1]
    packed = [tq.tq_pack_weight(_t(r), 4) for r in rs]
    wc = torch.cat([p[0] for p in packed], dim=0).contiguous()
    sw = torch.cat([p[1] for p in packed]).contiguous()
    lowrank = None
    if rk:
        lowrank = tq.tq_pack_lowrank_group([_t(a, torch.bfloat16) for a in l1s], [_t(a, torch.bfloat16) for a in l2s])
    ws = tq.linear_group_workspace(n, d, ms, rk, DEV)
    xt = _t(x, torch.bfloat16 if xdt == "bf16" else torch.float32)
    y = tq.tq_linear_group(xt, wc, sw, lowrank, ms, rk, y_dtype=y_dtype, ws=ws)
    torch.cuda.synchronize()
    return y, ws, wc


def _ws_parts(ws, n, d, ms, rk):
    """s_x, the activation codes and T (all layers' columns) from the group's workspace; its layout is the one of
    a single layer as wide as the group with the group's T width."""
    tc = _tcols(len(ms), rk)
    off = tq.tq_linear_workspace_offsets(n, d, int(sum(ms)), tc)
    b = ws.cpu().numpy()
    sx = b[off["s_x"]: off["s_x"] + 4 * n].view(np.float32)
    if n <= 32:
        codes = tqo.unpack_int4(b[off["x_codes"]: off["x_codes"] + n * d // 2].reshape(n, d // 2))
    else:
        codes = _int8_codes(b[off["x_codes"]: off["x_codes"] + n * d].reshape(n, d))
    t = None
    if rk:
        t = ws[off["T"]: off["T"] + n * tc * 2].view(torch.bfloat16).view(n, tc).float().cpu().numpy()
    return sx, codes, t


GCASES = [
    # (name, n, d, ms, r, x_kind, x_dtype, outliers)
    ("g2_n1_one_launch", 1, 1024, (256, 200), 32, "normal", "bf16", 2),
    ("g2_n2_one_launch", 2, 2048, (512, 256), 64, "normal", "bf16", 0),
    ("g3_n16_small_n", 16, 512, (256, 256, 128), 16, "normal", "f32", 2),
    ("g2_n8_d14336_two_launch", 8, 14336, (256, 96), 64, "student_t", "bf16", 0),
    ("g2_n40_tiles_ragged", 40, 544, (256, 272), 32, "normal", "bf16", 2),
    ("g3_n300_r32", 300, 1024, (512, 256, 256), 32, "normal", "bf16", 0),
    ("g2_n1030_one_pass_prologue", 1030, 512, (256, 256), 64, "normal", "bf16", 2),
    ("g4_n70_r0", 70, 512, (256, 256, 256, 64), 0, "normal", "bf16", 0),
    ("g8_n33", 33, 256, (256,) * 7 + (48,), 16, "normal", "bf16", 0),
    # one launch with blocks of 64 channels (more than 512 blocks of 16), the
    # second layer ragged
    ("g2_n12_one_launch_64ch", 12, 1024, (4096, 4112), 32, "normal", "bf16", 2),
]


@pytest.mark.parametrize("case", GCASES, ids=[c[0] for c in GCASES])
def test_linear_group(case):
    name, n, d, ms, rk, kind, xdt, nout = case
    print(f"case {name}", flush=True)
    c = draw_group_custom(n, d, ms, max(rk, 1), seed=3000 + n + d, x_kind=kind, x_dtype=xdt, outlier_count=nout,
                          outlier_scale=30.0)
    l1s = c["L1s"] if rk else None
    l2s = c["L2s"] if rk else None
    y, ws, wc = _run_group(c["X"], xdt, c["Rs"], l1s, l2s)
    ref = tqo.tq_linear_group_ref(c["X"], c["Rs"], l1s, l2s)
    sx, codes, t = _ws_parts(ws, n, d, ms, rk)
    assert np.array_equal(sx, ref["s_x"])
    assert np.array_equal(codes, ref["codes_x"])
    xc = _t(tqo.pack_int4(codes))
    yh = y.float().cpu().numpy().astype(np.float64)
    rp = _r_pad(rk)
    c0 = 0
    for g, (m, lay) in enumerate(zip(ms, ref["layers"])):
        acc = tq.tq_debug_accumulate(xc, wc[c0:c0 + m].contiguous(), d, 4)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy().astype(np.int64), lay["acc"]), g
        if rk:
            tg = t[:, g * rp: g * rp + rk]
            scale = np.abs(lay["T"]).max(axis=1, keepdims=True) + 1e-30
            assert (np.abs(tg - lay["T"]) / scale).max() <= 2e-2, g
        err = np.abs(yh[:, c0:c0 + m] - lay["Y"]).max()
        scale = np.abs(lay["Y"]).max()
        print(f"  layer {g}: max|Y-Yref|/max|Yref| = {err / max(scale, 1e-300):.3e}", flush=True)
        assert err <= TOL * scale, (g, err, scale)
        c0 += m


def test_group_of_one_is_the_single_layer():
    """One layer through the grouped entry point gives tq_linear's output bit for bit."""
    c = draw_group_custom(40, 512, [192], 32, seed=41)
    y, *_ = _run_group(c["X"], "bf16", c["Rs"], c["L1s"], c["L2s"], torch.float32)
    wc, sw = tq.tq_pack_weight(_t(c["Rs"][0]), 4)
    lowrank = tq.tq_pack_lowrank(_t(c["L1s"][0], torch.bfloat16), _t(c["L2s"][0], torch.bfloat16))
    y1 = tq.tq_linear(_t(c["X"], torch.bfloat16), wc, sw, lowrank, 192, 32, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, y1)


def test_group_graph_replay_matches_eager():
    """A grouped call captured in a HIP graph and replayed gives the eager output on every replay."""
    c = draw_group_custom(1, 1024, [256, 256], 64, seed=43)
    ms = [256, 256]
    packed = [tq.tq_pack_weight(_t(r), 4) for r in c["Rs"]]
    wc = torch.cat([p[0] for p in packed], dim=0).contiguous()
    sw = torch.cat([p[1] for p in packed]).contiguous()
    lowrank = tq.tq_pack_lowrank_group([_t(a, torch.bfloat16) for a in c["L1s"]],
                                       [_t(a, torch.bfloat16) for a in c["L2s"]])
    x = _t(c["X"], torch.bfloat16)
    ws = tq.linear_group_workspace(1, 1024, ms, 64, DEV)
    y = torch.empty((1, 512), dtype=torch.bfloat16, device=DEV)
    tq.tq_linear_group(x, wc, sw, lowrank, ms, 64, Y=y, ws=ws)
    torch.cuda.synchronize()
    eager = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tq.tq_linear_group(x, wc, sw, lowrank, ms, 64, Y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tq.tq_linear_group(x, wc, sw, lowrank, ms, 64, Y=y, ws=ws)
    for _ in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)

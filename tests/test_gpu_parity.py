"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bar: codes, scales and int32 accumulators bit-exact; Y within
max|Y - Y_ref| <= 1e-2 * max|Y_ref| (fp64 oracle); T = X L1 within one bf16
ulp plus the fp32 summation bound (tq_testutil).  The accumulators are those
of the kernels that produce Y: each layer call is repeated through its
accumulator-export entry point (tq_linear_debug, tq_linear_mp_bits_debug),
whose Y must equal the plain call's bit for bit.  Inputs come from the seeded
generators; expected values only from ``oracle``.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.tq_oracle as tqo  # noqa: E402
import rank_augmented_quantized_amd as tq  # noqa: E402
from tq_testutil import assert_t_tight  # noqa: E402
from workloads import WORKLOADS, draw_custom, draw_linear, draw_two_subspace, draw_two_subspace_custom  # noqa: E402

pytestmark = pytest.mark.gpu
TOL = 1e-2
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.load()  # fails loudly if libtq.so is missing


def _t(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def _x_tensor(x, x_dtype):
    return _t(x, torch.bfloat16 if x_dtype == "bf16" else torch.float32)


def _codes_np(t, k, bits):
    """Device code bytes -> int codes (oracle unpacking)."""
    b = t.cpu().numpy()
    return tqo.unpack_int4(b) if bits == 4 else b.view(np.int8).astype(np.int16)


def _assert_y(y_gpu, y_ref, what=""):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    ref = np.asarray(y_ref, dtype=np.float64)
    scale = np.abs(ref).max()
    err = np.abs(y - ref).max()
    print(f"  {what} max|Y-Yref|/max|Yref| = {err / max(scale, 1e-300):.3e}", flush=True)
    assert err <= TOL * scale, (what, err, scale)


# ----------------------------------------------------------------------------
# quantisation
# ----------------------------------------------------------------------------

def _golden_rows(d):
    rows = []
    import test_oracle_pins as pins

    for name, bits, vals, _, _ in pins.read_golden("quantizer_examples.txt"):
        if int(bits) != 4:
            continue
        v = [float(t) for t in vals.split()]
        rows.append(v + [0.0] * (d - len(v)))
    return np.array(rows, dtype=np.float32)


QCASES = [
    # (name, n, d, x_kind, x_dtype, outliers, bits)
    ("small_f32", 16, 512, "normal", "f32", 4, 4),
    ("bf16_ragged_outliers", 77, 4096, "normal", "bf16", 4, 4),
    ("bf16_plain_full_range", 37, 4096, "normal", "bf16", 0, 4),
    ("student_t_d14336", 5, 14336, "student_t", "bf16", 0, 4),
    ("int8_bf16", 33, 2048, "normal", "bf16", 4, 8),
    ("int8_f32_d48", 9, 48, "normal", "f32", 0, 8),
]


@pytest.mark.parametrize("case", QCASES, ids=[c[0] for c in QCASES])
def test_quantize_act_bitexact(case):
    name, n, d, kind, xdt, nout, bits = case
    print(f"case {name}", flush=True)
    x = draw_custom(n, d, 8, 1, seed=100 + n, x_kind=kind, x_dtype=xdt, outlier_count=nout, outlier_scale=30.0)["X"]
    x = x.copy()
    x[n // 2] = 0.0  # an all-zero row
    codes, sx = tq.tq_quantize_act(_x_tensor(x, xdt), bits)
    torch.cuda.synchronize()
    c_ref, s_ref = tqo.quantize_rows(x, bits)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    got = _codes_np(codes, d, bits)
    bad = np.argwhere(got != c_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"


def test_quantize_golden_rows_including_subnormal_scale():
    x = _golden_rows(32)
    codes, sx = tq.tq_quantize_act(_t(x), 4)
    torch.cuda.synchronize()
    c_ref, s_ref = tqo.quantize_rows(x, 4)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(_codes_np(codes, 32, 4), c_ref)


def test_quantize_rounding_boundaries():
    """Values placed exactly on and next to the half-integer boundaries of x/s."""
    rng = np.random.default_rng(5)
    n, d = 64, 512
    amax = rng.uniform(0.5, 40.0, size=n).astype(np.float32)
    s = (amax / np.float32(7)).astype(np.float32)
    half = (rng.integers(-7, 7, size=(n, d)) + 0.5).astype(np.float32)
    x = (half * s[:, None]).astype(np.float32)
    # nudge by -2..2 ulps
    bits = x.view(np.int32) + rng.integers(-2, 3, size=(n, d)).astype(np.int32)
    x = bits.view(np.float32)
    x = np.clip(x, -amax[:, None], amax[:, None])
    x[:, 0] = amax
    codes, sx = tq.tq_quantize_act(_t(x), 4)
    torch.cuda.synchronize()
    c_ref, s_ref = tqo.quantize_rows(x, 4)
    assert np.array_equal(sx.cpu().numpy(), s_ref)
    assert np.array_equal(_codes_np(codes, d, 4), c_ref)


# ----------------------------------------------------------------------------
# weight packing
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("d,m,dtype,bits", [(512, 512, "f32", 4), (4096, 200, "f32", 4), (1024, 96, "bf16", 4),
                                            (128, 300, "f32", 8), (8064, 64, "f32", 4)])
def test_pack_weight_bitexact(d, m, dtype, bits):
    print(f"case d={d} m={m} {dtype} bits={bits}", flush=True)
    case = draw_custom(4, d, m, 1, seed=d + m)
    w = case["R"].copy()
    w[:, 3] = 0.0  # an all-zero output channel
    if dtype == "bf16":
        from workloads import to_bf16_values

        w = to_bf16_values(w)
    codes, sw = tq.tq_pack_weight(_x_tensor(w, dtype), bits)
    torch.cuda.synchronize()
    c_ref, s_ref = tqo.quantize_weight(w, bits)
    assert np.array_equal(sw.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), tqo.pack_codes(c_ref, bits))


# ----------------------------------------------------------------------------
# exact integer accumulation (both main loops)
# ----------------------------------------------------------------------------

ACASES = [
    (1, 512, 16, 4), (16, 4096, 100, 4), (17, 512, 33, 4), (32, 14336, 48, 4), (33, 512, 130, 4),
    (200, 4064, 300, 4), (130, 8064, 257, 4), (64, 128, 200, 8), (5, 128, 40, 8), (300, 1024, 160, 8),
    # ragged last 128-k stage of the tile GEMM (8-bit: 16-byte chunks past k read as zeros)
    (40, 272, 96, 8), (70, 416, 64, 4),
]


@pytest.mark.parametrize("n,k,m,bits", ACASES)
def test_accumulate_bitexact(n, k, m, bits):
    print(f"case n={n} k={k} m={m} bits={bits}", flush=True)
    rng = np.random.default_rng(n * 7 + k + m)
    lo, hi = (-8, 7) if bits == 4 else (-128, 127)
    cx = rng.integers(lo, hi + 1, size=(n, k))
    cw = rng.integers(lo, hi + 1, size=(m, k))
    cx[0, :] = lo  # extreme magnitudes in one row / column
    cw[0, :] = lo
    acc = tq.tq_debug_accumulate(_t(tqo.pack_codes(cx, bits)), _t(tqo.pack_codes(cw, bits)), k, bits)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), tqo.int_matmul(cx, cw))


def _tile_order_int8(cx):
    """Activation codes as the tile GEMM takes them (include/tq.h, tq_debug_accumulate_i8): one int8 byte per code,
    within every 8 consecutive k the 4 codes of even k, then the 4 codes of odd k."""
    n, k = cx.shape
    g = cx.reshape(n, k // 8, 8)
    return np.concatenate([g[:, :, 0::2], g[:, :, 1::2]], axis=2).reshape(n, k).astype(np.int8)


@pytest.mark.parametrize("n,k,m", [(1, 512, 16), (33, 512, 130), (300, 1024, 160), (70, 416, 64), (200, 4064, 300),
                                   (4096, 256, 3584)])
def test_accumulate_i8_bitexact(n, k, m):
    """The tile GEMM's main loop on int8 activation codes (the layer's format), with the integer-export epilogue:
    every sum equals the exact product; 4096 x 3584 takes 224 tiles of 256 x 256."""
    print(f"case n={n} k={k} m={m}", flush=True)
    rng = np.random.default_rng(n * 5 + k + m)
    cx = rng.integers(-8, 8, size=(n, k))
    cw = rng.integers(-8, 8, size=(m, k))
    cx[0, :] = -8
    cw[0, :] = -8
    xi8 = torch.from_numpy(_tile_order_int8(cx)).to(DEV)
    acc = tq.tq_debug_accumulate_i8(xi8, _t(tqo.pack_codes(cw, 4)), k)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), tqo.int_matmul(cx, cw))


@pytest.mark.parametrize("n,k,m", [(33, 512, 130), (300, 1024, 160), (70, 416, 64), (4096, 256, 3584)])
def test_gemm_w4a4_both_activation_formats(n, k, m):
    """The residual product with its dequantising epilogue on nibble-packed and on int8 activation codes: the same
    bf16 Y bit for bit, and each element within the bf16 rounding of s_x s_w (C_x C_w^T) (relative 2^-8)."""
    print(f"case n={n} k={k} m={m}", flush=True)
    rng = np.random.default_rng(n * 3 + k + m)
    cx = rng.integers(-8, 8, size=(n, k))
    cw = rng.integers(-8, 8, size=(m, k))
    sx = rng.uniform(0.01, 2.0, size=n).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, size=m).astype(np.float32)
    wc, sxt, swt = _t(tqo.pack_codes(cw, 4)), _t(sx), _t(sw)
    y_p = tq.tq_debug_gemm_w4a4(_t(tqo.pack_codes(cx, 4)), True, sxt, wc, swt, k)
    y_8 = tq.tq_debug_gemm_w4a4(torch.from_numpy(_tile_order_int8(cx)).to(DEV), False, sxt, wc, swt, k)
    torch.cuda.synchronize()
    assert torch.equal(y_p, y_8)
    ref = sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] * tqo.int_matmul(cx, cw)
    y = y_p.float().cpu().numpy().astype(np.float64)
    assert (np.abs(y - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30).all()


# ----------------------------------------------------------------------------
# the layer on small shapes (several tiles, ragged tails)
# ----------------------------------------------------------------------------

def _run_linear(x, xdt, r_w, l1, l2, y_dtype=torch.bfloat16, want_acc=False):
    n, d = x.shape
    m = r_w.shape[1]
    r = 0 if l1 is None else l1.shape[1]
    wc, sw = tq.tq_pack_weight(_t(r_w), 4)
    lowrank = tq.tq_pack_lowrank(_t(l1, torch.bfloat16), _t(l2, torch.bfloat16)) if r else None
    ws = tq.linear_workspace(n, d, m, r, DEV)
    xt = _x_tensor(x, xdt)
    y = tq.tq_linear(xt, wc, sw, lowrank, m, r, y_dtype=y_dtype, ws=ws)
    torch.cuda.synchronize()
    if not want_acc:
        return y, ws, wc, sw
    acc = _linear_acc(xt, wc, sw, lowrank, m, r, y)
    return y, ws, wc, sw, acc


def _linear_acc(xt, wc, sw, lowrank, m, r, y):
    """The same call through tq_linear_debug: the kernels' int32 residual sums (n x m); its Y must be the plain
    call's, bit for bit."""
    n, d = xt.shape
    acc = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV)
    y2 = torch.empty_like(y)
    tq.tq_linear(xt, wc, sw, lowrank, m, r, Y=y2, ws=tq.linear_workspace(n, d, m, r, DEV), acc=acc)
    torch.cuda.synchronize()
    assert torch.equal(y2, y), "the accumulator-export call changed Y"
    return acc.cpu().numpy().astype(np.int64)


def _int8_codes(b):
    """Decode tq_linear's int8 activation codes for the tile GEMM (n > 32): one int8 byte per code; every 8-k group
    lists its 4 even-k codes, then its 4 odd-k codes (include/tq.h, tq_linear_workspace_offsets)."""
    n, d = b.shape
    v = b.view(np.int8).astype(np.int16).reshape(n, d // 8, 2, 4)
    out = np.empty((n, d // 8, 4, 2), np.int16)
    out[..., 0] = v[:, :, 0, :]
    out[..., 1] = v[:, :, 1, :]
    return out.reshape(n, d)


def _ws_codes(ws, n, d, m, r):
    """s_x and the activation codes tq_linear left in its workspace."""
    off = tq.tq_linear_workspace_offsets(n, d, m, r)
    b = ws.cpu().numpy()
    sx = b[off["s_x"]: off["s_x"] + 4 * n].view(np.float32)
    if n <= 32:
        xc = b[off["x_codes"]: off["x_codes"] + n * d // 2].reshape(n, d // 2)
        return sx, tqo.unpack_int4(xc)
    return sx, _int8_codes(b[off["x_codes"]: off["x_codes"] + n * d].reshape(n, d))


def _ws_packed_codes(ws, n, d, m, r):
    """The workspace activation codes as nibble-packed rows (device tensor), for tq_debug_accumulate."""
    _, codes = _ws_codes(ws, n, d, m, r)
    return _t(tqo.pack_int4(codes))


def _r_pad(r):
    p = 32
    while p < r:
        p *= 2
    return p if r else 0


def _assert_t(ws, x, l1, n, d, m, r, rows=None):
    """T = X L1 from the workspace against the fp64 product of the bf16-rounded X (tq_testutil bound)."""
    if not r:
        return
    rp = _r_pad(r)
    off = tq.tq_linear_workspace_offsets(n, d, m, r)["T"]
    t = ws[off: off + n * rp * 2].view(torch.bfloat16).view(n, rp).float().cpu().numpy()[:, :r]
    rows = np.arange(n) if rows is None else rows
    assert_t_tight(t[rows], np.asarray(x)[rows], l1)


LCASES = [
    # (name, n, d, m, r, x_kind, x_dtype, outliers)
    ("small_linear", 16, 512, 512, 16, "normal", "f32", 4),
    ("n1_ragged_m", 1, 512, 200, 16, "normal", "bf16", 4),
    ("n33_r0", 33, 256, 130, 0, "normal", "bf16", 0),
    ("n150_tiles", 150, 544, 272, 32, "normal", "bf16", 2),
    ("n200_r64", 200, 1024, 384, 64, "normal", "bf16", 0),
    ("n7_r96", 7, 1024, 100, 96, "student_t", "bf16", 0),
    ("n32_decode_edge", 32, 2048, 64, 64, "normal", "bf16", 2),
    ("n129_f32_out", 129, 512, 160, 32, "normal", "f32", 0),
    # d above the single-launch limit: the two-launch few-token path
    ("n4_d32800_two_launch", 4, 32800, 64, 32, "normal", "bf16", 3),
    ("n24_r256", 24, 1024, 48, 256, "normal", "bf16", 0),
    # many tokens: the one-pass prologue (16 rows per block, one per wave; rows
    # longer than 4096 take the two-kind prologue)
    ("n1030_d544_r128_fused", 1030, 544, 96, 128, "normal", "bf16", 2),
    ("n1100_f32_fused", 1100, 1024, 80, 32, "student_t", "f32", 0),
    ("n1040_r0_fused", 1040, 256, 64, 0, "normal", "bf16", 1),
    ("n1024_d8192_r32_long_rows", 1024, 8192, 64, 32, "normal", "bf16", 3),
    # 260 tiles of 256 x 256: the last 4 (two channel panels, the second
    # ragged) run as 256 x 128 tiles in a second launch
    ("n512_m33124_split_last_wave", 512, 256, 33124, 32, "normal", "bf16", 2),
    # 224 tiles of 256 x 256 with rows of 144 code bytes: the last 128-k
    # stage of each row is partial
    ("n4096_d288_full_tiles_ragged_k", 4096, 288, 3584, 32, "normal", "bf16", 2),
    # 128 x 128 tiles over long rows: 16, 64 and 17 stages of 128 k (the
    # last one partial, with fp32 Y)
    ("n100_d2048_tiles128", 100, 2048, 300, 32, "normal", "bf16", 2),
    ("n200_d8192_tiles128", 200, 8192, 520, 64, "normal", "bf16", 3),
    ("n70_d2080_ragged_k_f32_out", 70, 2080, 200, 32, "student_t", "bf16", 0),
    # one launch with blocks of 4 groups of 16 channels (more than 512 groups),
    # the last block with one group inside the layer
    ("n12_m8272_one_launch_64ch", 12, 2048, 8272, 32, "normal", "bf16", 2),
]


@pytest.mark.parametrize("case", LCASES, ids=[c[0] for c in LCASES])
def test_linear_small(case):
    name, n, d, m, r, kind, xdt, nout = case
    print(f"case {name}", flush=True)
    c = draw_custom(n, d, m, max(r, 1), seed=1000 + n + d, x_kind=kind, x_dtype=xdt, outlier_count=nout,
                    outlier_scale=30.0)
    l1 = c["L1"] if r else None
    l2 = c["L2"] if r else None
    ydt = torch.float32 if name.endswith("f32_out") else torch.bfloat16
    y, ws, wc, sw, acc_k = _run_linear(c["X"], xdt, c["R"], l1, l2, ydt, want_acc=True)
    ref = tqo.tq_linear_ref(c["X"], c["R"], l1, l2)
    sx, codes = _ws_codes(ws, n, d, m, r)
    assert np.array_equal(sx, ref["s_x"])
    assert np.array_equal(codes, ref["codes_x"])
    # the accumulators of the kernels that produced Y
    assert np.array_equal(acc_k, ref["acc"])
    # and the standalone integer GEMM on the same codes
    xc = _ws_packed_codes(ws, n, d, m, r)
    acc = tq.tq_debug_accumulate(xc, wc, d, 4)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), ref["acc"])
    _assert_t(ws, c["X"], l1, n, d, m, r)
    _assert_y(y, ref["Y"], name)


def test_linear_r0_is_pure_w4a4_and_deterministic():
    c = draw_custom(70, 512, 96, 16, seed=77)
    y0a, *_ = _run_linear(c["X"], "bf16", c["R"], None, None, torch.float32)
    y0b, *_ = _run_linear(c["X"], "bf16", c["R"], None, None, torch.float32)
    assert torch.equal(y0a, y0b)
    ref = tqo.tq_linear_ref(c["X"], c["R"])
    _assert_y(y0a, ref["Y"], "r0")
    # a zero L2 gives the same output as r = 0
    y1, *_ = _run_linear(c["X"], "bf16", c["R"], c["L1"], np.zeros_like(c["L2"]), torch.float32)
    assert torch.allclose(y1, y0a, rtol=0, atol=0)


def _sync_words(ws, n, d, m, r):
    """The hand-off words (4 KiB): word 0 the decode kernel's call counter, word 32 the wait-limit flag, every other
    word a counter that is zero between calls."""
    off = tq.tq_linear_workspace_offsets(n, d, m, r)["sync"]
    return ws[off: off + 4096].view(torch.int32).cpu().numpy()


def _one_launch(n, d, r):
    """Shapes of the decode kernel (include/tq.h): one or two tokens, d a multiple of 32 up to 16384, n d <= 16384,
    and at most 128 blocks computing partials of T (chunks of 512 k times r_pad / 16 column groups)."""
    nt = -(-d // 512) * (_r_pad(r) // 16)
    return n <= 2 and n * d <= 16384 and d <= 16384 and d % 32 == 0 and nt <= 128


def _fused_small(n, d, m, r):
    """Shapes of the one-launch few-token GEMM: up to 16 tokens, d up to 16384, not the decode kernel's, and a grid
    about resident at once: blocks of 16 channels up to 512 of them, else (d <= 4096) of 64 channels (the shapes
    here have at most a few hundred blocks, or far more than a GPU of 256 compute units holds)."""
    return (n <= 16 and d <= 16384 and not _one_launch(n, d, r)
            and (m // 16 <= 512 or (d <= 4096 and m // 64 < 600)))


@pytest.mark.parametrize("n,d,m,r", [(1, 4096, 300, 64), (2, 2048, 200, 64), (1, 4064, 64, 32), (2, 512, 40, 0),
                                     (2, 1024, 48, 256), (1, 14336, 64, 32), (1, 16384, 40, 32), (1, 16384, 40, 256), (2, 8192, 72, 32),
                                     (1, 96, 16, 32), (5, 2048, 200, 64), (3, 96, 16, 32), (16, 4096, 300, 64),
                                     (8, 14336, 72, 64), (11, 4064, 130, 256), (16, 8192, 64, 32), (9, 16384, 40, 32), (3, 16416, 40, 32),
                                     (8, 1024, 60000, 32), (16, 1024, 8256, 32), (5, 4096, 10000, 64),
                                     (24, 2048, 200, 64)])
def test_small_n_single_launch_handoff(n, d, m, r):
    """Up to 16 tokens run in one launch whose blocks wait for the codes and the partials of T that other blocks
    compute (17 .. 32 tokens, and rows longer than 16384, take two launches).  The decode kernel (one or two tokens) advances its call counter by one per call; both kernels leave
    the other words at zero (no wait gave up), and calls repeated on one workspace give identical outputs."""
    print(f"case n={n} d={d} m={m} r={r}", flush=True)
    c = draw_custom(n, d, m, max(r, 1), seed=90 + n)
    wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
    lowrank = tq.tq_pack_lowrank(_t(c["L1"], torch.bfloat16), _t(c["L2"], torch.bfloat16)) if r else None
    ws = tq.linear_workspace(n, d, m, r, DEV)
    x = _x_tensor(c["X"], "bf16")
    ys = []
    for call in range(4):
        if call == 0:  # which launches the call makes, by the library's own launch records
            tq.tq_profile_reset()
            tq.tq_profile_enable(True)
        ys.append(tq.tq_linear(x, wc, sw, lowrank, m, r, ws=ws))
        torch.cuda.synchronize()
        if call == 0:
            tq.tq_profile_enable(False)
            names = set(tq.tq_profile_read())
            tq.tq_profile_reset()
            assert names == ({"decode"} if _one_launch(n, d, r) else {"small_fused"} if _fused_small(n, d, m, r)
                             else {"prologue", "gemm_small_n"}), names
        w = _sync_words(ws, n, d, m, r)
        assert w[0] == (call + 1 if _one_launch(n, d, r) else 0)
        assert not w[1:].any()
    for y in ys[1:]:
        assert torch.equal(y, ys[0])
    ref = tqo.tq_linear_ref(c["X"], c["R"], c["L1"] if r else None, c["L2"] if r else None)
    _assert_y(ys[0], ref["Y"], f"n{n}")


@pytest.mark.parametrize("n,d,m,r", [(16, 512, 512, 16), (5, 14336, 80, 64)])
def test_one_launch_with_fp32_x(n, d, m, r):
    """fp32 X takes the one-launch few-token GEMM too (its producers read fp32 rows): one launch per call, codes,
    scales and every accumulator bit-exact, Y within the tolerance."""
    print(f"case n={n} d={d} m={m} r={r}", flush=True)
    c = draw_custom(n, d, m, r, seed=60 + n, x_dtype="f32")
    y, ws, wc, sw, acc_k = _run_linear(c["X"], "f32", c["R"], c["L1"], c["L2"], torch.bfloat16, want_acc=True)
    lowrank = tq.tq_pack_lowrank(_t(c["L1"], torch.bfloat16), _t(c["L2"], torch.bfloat16))
    xt = _x_tensor(c["X"], "f32")
    tq.tq_profile_reset()
    tq.tq_profile_enable(True)
    y2 = tq.tq_linear(xt, wc, sw, lowrank, m, r, ws=tq.linear_workspace(n, d, m, r, DEV))
    torch.cuda.synchronize()
    tq.tq_profile_enable(False)
    names = set(tq.tq_profile_read())
    tq.tq_profile_reset()
    assert names == {"small_fused"}, names
    assert torch.equal(y2, y)
    ref = tqo.tq_linear_ref(c["X"], c["R"], c["L1"], c["L2"])
    sx, codes = _ws_codes(ws, n, d, m, r)
    assert np.array_equal(sx, ref["s_x"])
    assert np.array_equal(codes, ref["codes_x"])
    assert np.array_equal(acc_k, ref["acc"])
    _assert_t(ws, c["X"], c["L1"], n, d, m, r)
    _assert_y(y, ref["Y"], f"fp32 X n={n}")


@pytest.mark.parametrize("n,d,m,r", [(1, 4096, 300, 64), (2, 8192, 40, 32), (16, 4096, 300, 64), (8, 14336, 72, 64),
                                     (12, 2048, 40, 32)])
def test_handoff_gives_up_loudly(n, d, m, r):
    """The one-launch paths' failure mode, forced from the host: the producer blocks never deliver (the decode
    kernel's tag its partials with the previous call's tag, the few-token GEMM's never signal) and the waits are
    limited to a few polls, so every wait gives up (every kernel still exits).  Y is then NaN everywhere and the
    flag word is set; later calls on that workspace keep writing NaN (the flag is sticky), and once the workspace is
    zero-filled a call gives the correct Y again."""
    print(f"case n={n} d={d} m={m} r={r}", flush=True)
    c = draw_custom(n, d, m, r, seed=70 + n)
    wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
    lowrank = tq.tq_pack_lowrank(_t(c["L1"], torch.bfloat16), _t(c["L2"], torch.bfloat16))
    ws = tq.linear_workspace(n, d, m, r, DEV)
    x = _x_tensor(c["X"], "bf16")
    y = torch.zeros((n, m), dtype=torch.bfloat16, device=DEV)
    tq.tq_debug_linear_handoff(x, wc, sw, lowrank, m, r, y, ws, spin=16, silent=True)
    torch.cuda.synchronize()
    assert torch.isnan(y).all()
    w = _sync_words(ws, n, d, m, r)
    assert w[32] != 0 and not np.delete(w, [0, 32]).any() and w[0] == (1 if _one_launch(n, d, r) else 0)
    y2 = tq.tq_linear(x, wc, sw, lowrank, m, r, ws=ws)
    torch.cuda.synchronize()
    assert torch.isnan(y2).all()
    ws.zero_()
    y3 = tq.tq_linear(x, wc, sw, lowrank, m, r, ws=ws)
    torch.cuda.synchronize()
    ref = tqo.tq_linear_ref(c["X"], c["R"], c["L1"], c["L2"])
    _assert_y(y3, ref["Y"], "after zero-fill")
    assert not _sync_words(ws, n, d, m, r)[1:].any()


@pytest.mark.parametrize("n,d,m,r", [(1, 2048, 300, 64), (16, 1024, 200, 32), (40, 512, 96, 32),
                                     (1030, 512, 80, 32), (100, 2048, 300, 32)])
def test_graph_replay_matches_eager(n, d, m, r):
    """tq_linear captured in a HIP graph (as a serving loop would run it): every replay, with eager calls and
    synchronisations in between, gives the eager output bit for bit and leaves the hand-off words at zero."""
    print(f"case n={n} d={d} m={m} r={r}", flush=True)
    c = draw_custom(n, d, m, r, seed=500 + n)
    wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
    lowrank = tq.tq_pack_lowrank(_t(c["L1"], torch.bfloat16), _t(c["L2"], torch.bfloat16))
    x = _x_tensor(c["X"], "bf16")
    ws_e = tq.linear_workspace(n, d, m, r, DEV)
    y_e = tq.tq_linear(x, wc, sw, lowrank, m, r, ws=ws_e)
    torch.cuda.synchronize()
    ws_g = tq.linear_workspace(n, d, m, r, DEV)
    y_g = torch.empty_like(y_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tq.tq_linear(x, wc, sw, lowrank, m, r, Y=y_g, ws=ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tq.tq_linear(x, wc, sw, lowrank, m, r, Y=y_g, ws=ws_g)
    for rep in range(3):
        y_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {rep}"
        assert not _sync_words(ws_g, n, d, m, r)[1:].any()
        y_again = tq.tq_linear(x, wc, sw, lowrank, m, r, ws=ws_e)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y_again, y_e)


def test_workspace_reused_across_shapes():
    """One workspace, zero-filled once, serves calls of different shapes in turn (the prologue's cross-block
    counters, the one-launch few-token GEMM, the decode kernel): every call equals the same call on a fresh
    workspace bit for bit, since every counter sits at a fixed offset and is zero again after each call."""
    shapes = [(300, 1024, 512, 32), (40, 4096, 256, 32), (200, 1024, 384, 64), (12, 4096, 200, 64), (1, 4096, 300, 64),
              (100, 2048, 300, 32), (70, 2080, 200, 32)]
    big = max(tq.tq_linear_workspace_bytes(*sh) for sh in shapes)
    ws = torch.zeros(big, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        for i, (n, d, m, r) in enumerate(shapes):
            print(f"pass {rep} case n={n} d={d} m={m} r={r}", flush=True)
            c = draw_custom(n, d, m, r, seed=40 + i)
            wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
            lowrank = tq.tq_pack_lowrank(_t(c["L1"], torch.bfloat16), _t(c["L2"], torch.bfloat16))
            x = _x_tensor(c["X"], "bf16")
            y_fresh = tq.tq_linear(x, wc, sw, lowrank, m, r, ws=tq.linear_workspace(n, d, m, r, DEV))
            y = tq.tq_linear(x, wc, sw, lowrank, m, r, ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(y, y_fresh), (rep, i)


def test_small_n_and_tile_paths_agree():
    c = draw_custom(33, 1024, 128, 32, seed=78)
    y33, *_ = _run_linear(c["X"], "bf16", c["R"], c["L1"], c["L2"], torch.float32)
    y32, *_ = _run_linear(c["X"][:32], "bf16", c["R"], c["L1"], c["L2"], torch.float32)
    a = y33[:32].cpu().numpy()
    b = y32.cpu().numpy()
    assert np.abs(a - b).max() <= 1e-5 * np.abs(a).max()


# ----------------------------------------------------------------------------
# the workloads at full size (sampled outputs)
# ----------------------------------------------------------------------------

def _sample(n, m, rng, k_rows=24, k_cols=48):
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=min(n, k_rows))]))
    cols = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, size=min(m, k_cols))]))
    return rows, cols


WCASES = [("attn_proj", 4096, True), ("attn_proj", 4096, False), ("mlp_gate_up", 1, True),
          ("mlp_gate_up", 16, True), ("mlp_gate_up", 256, True), ("mlp_gate_up", 4096, True),
          ("mlp_gate_up", 16, False), ("mlp_down", 1, True), ("mlp_down", 8, True), ("mlp_down", 32, True),
          ("small", 16, True)]


@pytest.mark.parametrize("wl,n,outl", WCASES, ids=[f"{w}-n{n}-{'outliers' if o else 'plain'}" for w, n, o in WCASES])
def test_linear_workload(wl, n, outl):
    """The workloads at full size, compared in full: every code and scale, every int32 accumulator of the kernels
    that produced Y, T, and every element of Y."""
    w = WORKLOADS[wl]
    print(f"case {w.title} n={n} outliers={outl}", flush=True)
    c = draw_linear(w, n=n, outliers=outl)
    d, m, r = w.d, w.m, w.r
    y, ws, wc, sw, acc_k = _run_linear(c["X"], w.x_dtype, c["R"], c["L1"], c["L2"], want_acc=True)
    ref = tqo.tq_linear_ref(c["X"], c["R"], c["L1"], c["L2"])
    sx, codes = _ws_codes(ws, n, d, m, r)
    assert np.array_equal(sx, ref["s_x"])
    assert np.array_equal(codes, ref["codes_x"])
    assert np.array_equal(sw.cpu().numpy(), ref["s_w"])
    assert np.array_equal(wc.cpu().numpy(), tqo.pack_int4(ref["codes_w"]))
    bad = np.argwhere(acc_k != ref["acc"])
    assert bad.size == 0, f"{len(bad)} accumulators differ, first {bad[:5].tolist()}"
    _assert_t(ws, c["X"], c["L1"], n, d, m, r)
    _assert_y(y, ref["Y"], f"{wl} n={n}")


# ----------------------------------------------------------------------------
# two-subspace layer
# ----------------------------------------------------------------------------

def _run_mp(xrot, wrot, d_hi):
    """The two-subspace layer, then the same call through tq_linear_mp_bits_debug: returns Y and the kernel's
    int32 sums of both subspaces (Y of the export call must equal Y bit for bit)."""
    n, d = xrot.shape
    m = wrot.shape[1]
    dl = d - d_hi
    wlc, swl = tq.tq_pack_weight(_t(np.ascontiguousarray(wrot[:dl])), 4) if dl else (None, None)
    whc, swh = tq.tq_pack_weight(_t(np.ascontiguousarray(wrot[dl:])), 8) if d_hi else (None, None)
    xt = _t(xrot, torch.bfloat16)
    y = tq.tq_linear_mp(xt, d_hi, wlc, swl, whc, swh, m)
    acc_l = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV)
    acc_h = torch.full((n, m), -(2 ** 31), dtype=torch.int32, device=DEV) if d_hi else None
    y2 = tq.tq_linear_mp(xt, d_hi, wlc, swl, whc, swh, m, acc_l=acc_l, acc_h=acc_h)
    torch.cuda.synchronize()
    assert torch.equal(y2, y), "the accumulator-export call changed Y"
    acc_l = acc_l.cpu().numpy().astype(np.int64)
    acc_h = acc_h.cpu().numpy().astype(np.int64) if d_hi else np.zeros((n, m), np.int64)
    return y, acc_l, acc_h


def _assert_mp_acc(acc_l, acc_h, ref, rows=None, cols=None):
    if rows is not None:
        acc_l, acc_h = acc_l[np.ix_(rows, cols)], acc_h[np.ix_(rows, cols)]
    assert np.array_equal(acc_l, ref["acc_l"])
    assert np.array_equal(acc_h, ref["acc_h"])


@pytest.mark.parametrize("n,d,m,dh", [(40, 512, 96, 64), (130, 1024, 272, 128), (16, 256, 64, 0),
                                      (70, 256, 80, 256), (9, 8192, 48, 128), (70, 1024, 80, 512),
                                      (300, 1024, 200, 384), (512, 1024, 28672, 512), (512, 1024, 28672, 128),
                                      (1, 128, 32, 32), (40, 560, 96, 48), (70, 1056, 80, 32), (33, 608, 64, 96)])
def test_linear_mp_small(n, d, m, dh):
    """Ragged tails; high subspaces of 0 .. 512 columns, including widths that are not a multiple of 64; the
    256 x 256 tile (n = 512, m = 28672)."""
    print(f"case mp n={n} d={d} m={m} d_hi={dh}", flush=True)
    c = draw_two_subspace_custom(n, d, m, dh, seed=n + d + m, outlier_count=2, block=128 if d % 128 == 0 else 16)
    y, acc_l, acc_h = _run_mp(c["Xrot"], c["Wrot"], dh)
    rows, cols = (None, None) if m < 4096 else _sample(n, m, np.random.default_rng(n), 64, 512)
    ref = tqo.tq_linear_mp_ref(c["Xrot"], c["Wrot"], dh, rows=rows, cols=cols)
    _assert_mp_acc(acc_l, acc_h, ref, rows, cols)
    if rows is not None:
        y = y[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)]
    _assert_y(y, ref["Y"], f"mp n={n} d={d} dh={dh}")


def test_linear_mp_workload():
    """The 70B MLP two-subspace shape (8192 x 8192 x 28672, 128-dim 8-bit subspace), compared in full: every
    int32 sum of both subspaces and every element of Y."""
    w = WORKLOADS["two_subspace"]
    print(f"case {w.title}", flush=True)
    c = draw_two_subspace(w)
    y, acc_l, acc_h = _run_mp(c["Xrot"], c["Wrot"], w.d_hi)
    ref = tqo.tq_linear_mp_ref(c["Xrot"], c["Wrot"], w.d_hi)
    _assert_mp_acc(acc_l, acc_h, ref)
    del acc_l, acc_h
    _assert_y(y, ref["Y"], "two_subspace")

"""tq_linear_noalloc -- tq_linear with the library's own device scratch instead of a caller workspace -- against
tq_linear on the same inputs, through the C ABI: calls in a row on one device, each on a smaller input than the one
before (so each finds the scratch as the previous, larger call left it), every Y equal to tq_linear's bit for bit
and within max|Y - Y_ref| <= 1e-2 * max|Y_ref| of the fp64 oracle; a size past the scratch is refused before any
launch."""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.tq_oracle as tqo  # noqa: E402
import rank_augmented_quantized_amd as tq  # noqa: E402
from workloads import draw_custom  # noqa: E402

pytestmark = pytest.mark.gpu
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


# (n, d, m, r): the tile GEMM after the one-pass prologue; the prologue whose T partials are summed across blocks
# through counters; the one-launch decode kernel with its hand-off words; the small-n GEMM without low-rank factors
CALLS = [(300, 1024, 512, 32), (40, 4096, 256, 32), (1, 1024, 512, 64), (5, 512, 96, 0)]


def test_noalloc_calls_in_a_row_match_tq_linear():
    for i, (n, d, m, r) in enumerate(CALLS):
        print(f"call {i}: n={n} d={d} m={m} r={r}", flush=True)
        c = draw_custom(n, d, m, max(r, 1), seed=900 + i)
        wc, sw = tq.tq_pack_weight(_t(c["R"]), 4)
        lr = tq.tq_pack_lowrank(_t(c["L1"], torch.bfloat16), _t(c["L2"], torch.bfloat16)) if r else None
        x = _t(c["X"], torch.bfloat16)
        y_ref = tq.tq_linear(x, wc, sw, lr, m, r)
        y = torch.full_like(y_ref, float("nan"))
        tq.tq_linear_noalloc(x, wc, sw, lr, m, r, y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"call {i} differs from tq_linear"
        ref = tqo.tq_linear_ref(c["X"], c["R"], c["L1"] if r else None, c["L2"] if r else None)
        err = np.abs(y.float().cpu().numpy().astype(np.float64) - ref["Y"]).max()
        assert err <= 1e-2 * np.abs(ref["Y"]).max(), (i, err)


def test_noalloc_refuses_sizes_past_its_scratch():
    n, d, m, r = 8192, 8192, 256, 32
    assert tq.tq_linear_workspace_bytes(n, d, m, r) > tq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((n, d), dtype=torch.bfloat16, device=DEV)
    wc = torch.zeros((m, d // 2), dtype=torch.uint8, device=DEV)
    sw = torch.zeros(m, dtype=torch.float32, device=DEV)
    lr = torch.zeros(tq.load().tq_lowrank_bytes(d, m, r), dtype=torch.uint8, device=DEV)
    y = torch.zeros((n, m), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tq.TQError) as e:
        tq.tq_linear_noalloc(x, wc, sw, lr, m, r, y)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert not y.any()  # nothing was enqueued

"""The two measurement kernels behind the roofline ceilings do the work they are timed for.

tq_debug_mfma_ceiling: every wave chains 8 independent int8 32x32x32 products of fixed register operands; the sum
of all accumulator elements of a wave is iters x 8 x sum over k of (column sum of A at k) x (row sum of B at k),
computed here from the operand bytes each lane supplies (lanes l and l + 32 hold the two k halves of row l of A and
column l of B).  tq_debug_stream_read: each block XORs the 16-byte units of its slab, so the words are the XOR of
contiguous slabs of the buffer.
"""

from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import rank_augmented_quantized_amd as tq  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.load()


def _lane_bytes(vals):
    """The 16 int8 operand bytes of each of the 64 lanes: 4 little-endian int32 words per lane."""
    w = np.stack([np.asarray(v, dtype=np.int64) for v in vals], axis=1).astype(np.int32)  # [64, 4]
    return w.view(np.int8).reshape(64, 16).astype(np.int64)


@pytest.mark.parametrize("iters,blocks", [(1, 1), (5, 3)])
def test_mfma_ceiling_products(iters, blocks):
    lane = np.arange(64)
    a = _lane_bytes([lane, lane + 1, lane + 2, lane + 3])
    b = _lane_bytes([3 * lane, lane, np.full(64, 7), lane ^ 5])
    per_k = a[:32].sum(0) * b[:32].sum(0) + a[32:].sum(0) * b[32:].sum(0)
    want = (iters * 8 * int(per_k.sum())) % (1 << 32)
    out = torch.zeros(512 * blocks, dtype=torch.int32, device="cuda")
    tq.tq_debug_mfma_ceiling(out, iters, blocks)
    torch.cuda.synchronize()
    per_wave = out.cpu().numpy().astype(np.int64).reshape(blocks * 8, 64).sum(1) % (1 << 32)
    assert (per_wave == want).all(), (per_wave[:4], want)


def test_stream_read_xor():
    g = torch.Generator().manual_seed(7)
    buf = torch.randint(-(1 << 31), (1 << 31) - 1, (1 << 16,), dtype=torch.int32, generator=g)
    blocks = 4
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    tq.tq_debug_stream_read(buf.cuda(), out, blocks)
    torch.cuda.synchronize()
    slabs = buf.numpy().view(np.uint32).reshape(blocks, -1)
    want = np.bitwise_xor.reduce(slabs, axis=1)
    assert (out.cpu().numpy().view(np.uint32) == want).all()

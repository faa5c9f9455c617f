"""CPU oracle for the rank-augmented W4A4 linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

It evaluates the plain definition of the layer, step by step, in numpy:

* symmetric integer quantiser -- TwinQuant notes ("TwinQuant: Learnable
  Subspace Decomposition for W4A4 LLM Quantization"), section 02 Background,
  the quantization formula Q_x = round(x/s), s = max|X|/q_max; CoQuant
  ("CoQuant: Joint Weight-Activation Subspace Projection for Mixed-Precision
  LLMs"), Eq. 1 with zero-point z = 0 and s = max|X|/(2^(N-1)-1);
  granularity per token for activations and per output channel for weights
  (CoQuant, experimental protocol following ResQ);
* the low-rank plus residual form Y = Q(X)Q(R) + X.L1.L2 -- TwinQuant notes,
  section 02.A (SVDQuant decomposition), with the low-rank branch fed by the
  unquantised activations;
* exact integer accumulation of the residual product -- TwinQuant notes,
  section 02 (note on INT32 accumulation) and section 04.C, Figure 4;
* the two-subspace mixed-precision output -- CoQuant Eq. 3-9;
* layers that share one input, grouped -- CoQuant, the grouping paragraph
  around Eq. 14;
* the fully quantised low-rank branch Q(X)[Q(U)Q(V) + Q(R)] with the first
  stage's integer result re-quantised per token -- TwinQuant notes, the
  error expression of section 04.A and the fused two-stage low-rank pipeline
  of section 04.C;
* per-token asymmetric activations (a zero-point per token) for the
  two-subspace layer and for the rank-augmented layer -- CoQuant Eq. 1 with
  z != 0 and the experimental protocol (per-token asymmetric activations,
  per-channel symmetric weights).

Readings of points the pages leave open (each one is also listed in the
design notes): q_max = 7 / 127; "round" is round-half-to-even; the scale is
the fp32 quotient fl(max|row| / q_max) and each code is rne(fl(x / s)) with an
IEEE fp32 division; a row whose scale is 0 gets codes 0; codes are clamped to
[-2^(N-1), 2^(N-1)-1]; the final output is evaluated in fp64.

Codes are stored as two's-complement nibbles, two per byte, the even index of
each pair in the low nibble; 8-bit codes are plain int8.  Every function is
pinned by the CPU tests (worked examples, brute force against exact rational
arithmetic, invariants, lossless special cases); none is "parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "qmax_of",
    "quantize_rows",
    "quantize_weight",
    "pack_int4",
    "unpack_int4",
    "pack_codes",
    "int_matmul",
    "lowrank_branch",
    "tq_linear_ref",
    "tq_linear_mp_ref",
    "hadamard",
    "block_rotation",
    "rotate",
    "subspace_split",
    "requantize_lowrank",
    "tq_linear_qlr_ref",
    "quantize_rows_asym",
    "tq_linear_mp_asym_ref",
    "tq_linear_asym_ref",
]


def qmax_of(bits: int) -> int:
    """Largest code of the symmetric N-bit quantiser: 2^(N-1) - 1 (CoQuant Eq. 1)."""
    if bits not in (2, 3, 4, 5, 6, 7, 8):
        raise ValueError(f"unsupported bit width {bits}")
    return (1 << (bits - 1)) - 1


def quantize_rows(a, bits: int = 4):
    """Per-row symmetric quantisation (TwinQuant notes section 02; CoQuant Eq. 1).

    For each row: amax = max|a_row| (exact), s = fl32(amax / q_max), and each
    code c = clip(rint(fl32(a / s)), -2^(bits-1), q_max) with round half to
    even.  A row with s == 0 gets s = 0 and codes 0.

    Returns (codes int16 [rows, K], scales float32 [rows]).
    """
    a = np.asarray(a, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError("quantize_rows expects a 2-D array")
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input is outside the quantiser's contract")
    qmax = qmax_of(bits)
    amax = np.max(np.abs(a), axis=1) if a.shape[1] else np.zeros(a.shape[0], np.float32)
    s = (amax.astype(np.float32) / np.float32(qmax)).astype(np.float32)
    codes = np.zeros(a.shape, dtype=np.int16)
    live = s > 0
    if np.any(live):
        q = (a[live] / s[live][:, None]).astype(np.float32)  # IEEE fp32 division
        codes[live] = np.clip(np.rint(q), -(qmax + 1), qmax).astype(np.int16)
    return codes, s


def quantize_weight(w, bits: int = 4):
    """Per-output-channel symmetric quantisation of a d x m weight (Y = X W).

    Output channel j is column j of W (CoQuant Eq. 2 layout); it is quantised
    as one row of W^T.  Returns (codes int16 [m, d] -- K contiguous per output
    channel, scales float32 [m]).
    """
    w = np.asarray(w, dtype=np.float32)
    return quantize_rows(np.ascontiguousarray(w.T), bits)


def pack_int4(codes):
    """Pack codes in [-8, 7] two per byte: even index -> low nibble, odd -> high."""
    c = np.asarray(codes)
    if c.shape[-1] % 2:
        raise ValueError("the packed dimension must be even")
    if c.size and (c.min() < -8 or c.max() > 7):
        raise ValueError("int4 codes must lie in [-8, 7]")
    u = (c.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed):
    """Inverse of pack_int4: two's-complement nibbles back to int16 codes."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_codes(codes, bits: int):
    """Storage bytes of a code matrix: nibbles for 4 bits, int8 bytes for 8 bits."""
    if bits == 4:
        return pack_int4(codes)
    if bits == 8:
        return np.asarray(codes).astype(np.int8).view(np.uint8)
    raise ValueError("storage is defined for 4 and 8 bits")


def int_matmul(cx, cw):
    """Exact integer product acc[i, j] = sum_k cx[i, k] * cw[j, k].

    Evaluated as an fp64 matrix product of integer-valued arrays; that is exact
    because every partial sum is an integer below 2^53 in magnitude, which is
    asserted from the operands' ranges.  Returns int64.
    """
    cx = np.asarray(cx)
    cw = np.asarray(cw)
    if cx.shape[1] != cw.shape[1]:
        raise ValueError("inner dimensions differ")
    k = cx.shape[1]
    bx = int(np.max(np.abs(cx))) if cx.size else 0
    bw = int(np.max(np.abs(cw))) if cw.size else 0
    if k * bx * bw >= 2 ** 53:
        raise ValueError("integer product would not be exact in fp64")
    acc = cx.astype(np.float64) @ cw.astype(np.float64).T
    return acc.astype(np.int64)


def lowrank_branch(x, l1, l2):
    """Low-rank branch (X . L1) . L2 in fp64 from the unquantised activations.

    TwinQuant notes section 02.A (the U V term of the SVDQuant form) and
    section 04.C (the two-stage product U then V).
    """
    t = np.asarray(x, dtype=np.float64) @ np.asarray(l1, dtype=np.float64)
    return t, t @ np.asarray(l2, dtype=np.float64)


def tq_linear_ref(x, r, l1=None, l2=None, rows=None, cols=None, bits: int = 4):
    """Reference output of the rank-augmented quantised linear layer.

    Y = s_x s_w^T (.) (C_x C_w^T) + (X L1) L2          (all in fp64)

    with C_x, s_x the per-token codes and scales of X, C_w, s_w the
    per-output-channel codes and scales of R, following the TwinQuant notes
    section 02.A decomposition and the single shared epilogue of section
    04.C.  ``rows`` / ``cols`` restrict the evaluation to a subset of tokens /
    output channels (quantisation is row- and column-local, so the sampled
    values equal the full computation's).
    """
    x = np.asarray(x, dtype=np.float32)
    r = np.asarray(r, dtype=np.float32)
    if rows is not None:
        x = x[np.asarray(rows)]
    if cols is not None:
        r = r[:, np.asarray(cols)]
        if l2 is not None:
            l2 = np.asarray(l2)[:, np.asarray(cols)]
    cw, s_w = quantize_weight(r, bits)
    cx, s_x = quantize_rows(x, bits)
    acc = int_matmul(cx, cw)
    y = (s_x.astype(np.float64)[:, None] * s_w.astype(np.float64)[None, :]) * acc.astype(np.float64)
    t = None
    if l1 is not None and np.asarray(l1).shape[1] > 0:
        t, ylr = lowrank_branch(x, l1, l2)
        y = y + ylr
    return {"codes_x": cx, "s_x": s_x, "codes_w": cw, "s_w": s_w, "acc": acc, "T": t, "Y": y}


def tq_linear_group_ref(x, rs, l1s=None, l2s=None, rows=None, bits: int = 4):
    """Reference output of G layers that share one input.

    The CoQuant notes group the linear layers whose input activations are
    identical (query/key/value, gate/up; the paragraph around Eq. 14).  Layer
    g is the layer of ``tq_linear_ref`` on the same X with its own weight
    rs[g] (d x m_g) and factors l1s[g], l2s[g]; the outputs sit side by side,
    layer g in the m_g columns after those of layers 0 .. g-1.  X is
    quantised once: its codes and scales are every layer's.
    """
    outs = []
    for g, r in enumerate(rs):
        l1 = None if l1s is None else l1s[g]
        l2 = None if l2s is None else l2s[g]
        outs.append(tq_linear_ref(x, r, l1, l2, rows=rows, bits=bits))
    y = np.concatenate([o["Y"] for o in outs], axis=1)
    t = None if outs[0]["T"] is None else np.concatenate([o["T"] for o in outs], axis=1)
    return {"codes_x": outs[0]["codes_x"], "s_x": outs[0]["s_x"], "layers": outs, "T": t, "Y": y}


def requantize_lowrank(acc1, s_u, bits: int = 4):
    """Per-token re-quantisation of the first low-rank stage (TwinQuant notes,
    section 04.C: the integer result of Q(X) Q(U) is brought back to ``bits``
    before it meets Q(V)).

    acc1 is the exact integer product C_x C_u^T (tokens x r).  The real-valued
    stage is s_x[i] * s_u[j] * acc1[i, j]; the token's own factor s_x[i] is
    common to its whole row, so it is kept outside and the row that is
    quantised is t[i, j] = fl32(fl32(acc1[i, j]) * s_u[j]) (acc1 is exact in
    fp32 below 2^24 in magnitude, which is asserted).  t is quantised per
    token by ``quantize_rows``, so the stage's scale is s_x * s_t.

    Returns (t fp32, codes int16, s_t fp32).
    """
    acc1 = np.asarray(acc1)
    if acc1.size and int(np.max(np.abs(acc1))) >= 2 ** 24:
        raise ValueError("first-stage sum not exact in fp32")
    t = (acc1.astype(np.float32) * np.asarray(s_u, dtype=np.float32)[None, :]).astype(np.float32)
    ct, s_t = quantize_rows(t, bits)
    return t, ct, s_t


def tq_linear_qlr_ref(x, r, u, v, rows=None, cols=None, bits: int = 4):
    """Layer with both branches quantised (TwinQuant notes, section 04.A error
    expression Q(X)[Q(U)Q(V) + Q(R)], kernel of section 04.C, Figure 4):

        acc  = C_x C_w^T                     residual product, exact
        acc1 = C_x C_u^T                     first low-rank stage, exact
        (t, C_t, s_t) = requantize_lowrank(acc1, s_u)
        acc2 = C_t C_v^T                     second low-rank stage, exact
        Y = s_x s_w^T (.) acc + (s_x s_t) s_v^T (.) acc2     (fp64)

    X (n x d) per token, R (d x m), U (d x r) and V (r x m) per output
    channel (column), all symmetric at ``bits``.  ``rows`` / ``cols`` restrict
    the evaluation to some tokens / output channels (every step is row- or
    column-local, so the sampled values equal the full computation's).
    """
    x = np.asarray(x, dtype=np.float32)
    r = np.asarray(r, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    if rows is not None:
        x = x[np.asarray(rows)]
    if cols is not None:
        r = r[:, np.asarray(cols)]
        v = v[:, np.asarray(cols)]
    cx, s_x = quantize_rows(x, bits)
    cw, s_w = quantize_weight(r, bits)
    acc = int_matmul(cx, cw)
    cu, s_u = quantize_weight(u, bits)
    acc1 = int_matmul(cx, cu)
    t, ct, s_t = requantize_lowrank(acc1, s_u, bits)
    cv, s_v = quantize_weight(v, bits)
    acc2 = int_matmul(ct, cv)
    sx = s_x.astype(np.float64)[:, None]
    y = sx * s_w.astype(np.float64)[None, :] * acc.astype(np.float64)
    y = y + (sx * s_t.astype(np.float64)[:, None]) * s_v.astype(np.float64)[None, :] * acc2.astype(np.float64)
    return {"codes_x": cx, "s_x": s_x, "acc": acc, "codes_u": cu, "s_u": s_u, "acc1": acc1, "t": t,
            "codes_t": ct, "s_t": s_t, "codes_v": cv, "s_v": s_v, "acc2": acc2, "Y": y}


def tq_linear_mp_ref(xrot, wrot, d_hi: int, rows=None, cols=None, bits_lo: int = 4, bits_hi: int = 8):
    """Two-subspace mixed-precision output (CoQuant Eq. 9).

    Y = Q_l(X_l) Q_l(W_l) + Q_h(X_h) Q_h(W_h), where X_l / X_h are the first
    d - d_hi / last d_hi columns of the rotated activations and W_l / W_h the
    matching rows of the rotated weight (Eq. 6-7 after the rotation of Eq. 3).
    Q_l quantises per token / per output channel at ``bits_lo``; Q_h at
    ``bits_hi``; each subspace has its own scales.
    """
    xrot = np.asarray(xrot, dtype=np.float32)
    wrot = np.asarray(wrot, dtype=np.float32)
    d = xrot.shape[1]
    if not 0 <= d_hi <= d:
        raise ValueError("d_hi out of range")
    if rows is not None:
        xrot = xrot[np.asarray(rows)]
    if cols is not None:
        wrot = wrot[:, np.asarray(cols)]
    dl = d - d_hi
    out = {}
    y = np.zeros((xrot.shape[0], wrot.shape[1]), dtype=np.float64)
    for tag, xs, ws, bits in (("l", xrot[:, :dl], wrot[:dl], bits_lo), ("h", xrot[:, dl:], wrot[dl:], bits_hi)):
        cx, s_x = quantize_rows(xs, bits)
        cw, s_w = quantize_weight(ws, bits)
        acc = int_matmul(cx, cw)
        y = y + (s_x.astype(np.float64)[:, None] * s_w.astype(np.float64)[None, :]) * acc.astype(np.float64)
        out.update({f"codes_x{tag}": cx, f"s_x{tag}": s_x, f"codes_w{tag}": cw, f"s_w{tag}": s_w, f"acc_{tag}": acc})
    out["Y"] = y
    return out


def quantize_rows_asym(a, bits: int = 4):
    """Per-row asymmetric quantisation (CoQuant Eq. 1 with a zero-point: the
    dequantised value is u s + z, u the rounded and clipped (x - z) / s).

    The scale and zero-point follow the row's range: z = min(row) and
    s = fl32(fl32(max - min) / (2^N - 1)); each code is
    u = clip(rint(fl32(fl32(x - z) / s)), 0, 2^N - 1) with IEEE fp32
    subtraction and division and round half to even.  A constant row has
    s = 0 and codes 0 (it dequantises to z exactly).

    Returns (u int16 [rows, K] in [0, 2^N - 1], s float32 [rows], z float32 [rows]).
    """
    a = np.asarray(a, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError("quantize_rows_asym expects a 2-D array")
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input is outside the quantiser's contract")
    qm = (1 << bits) - 1
    if a.shape[1] == 0:
        z = np.zeros(a.shape[0], np.float32)
        return np.zeros(a.shape, np.int16), z.copy(), z
    mn = a.min(axis=1)
    mx = a.max(axis=1)
    s = ((mx - mn).astype(np.float32) / np.float32(qm)).astype(np.float32)
    u = np.zeros(a.shape, dtype=np.int16)
    live = s > 0
    if np.any(live):
        dlt = (a[live] - mn[live][:, None]).astype(np.float32)  # fl32(x - z)
        q = (dlt / s[live][:, None]).astype(np.float32)          # IEEE fp32 division
        u[live] = np.clip(np.rint(q), 0, qm).astype(np.int16)
    return u, s, mn.astype(np.float32)


def tq_linear_mp_asym_ref(xrot, wrot, d_hi: int, rows=None, cols=None, bits_lo: int = 4, bits_hi: int = 8):
    """The two-subspace output (CoQuant Eq. 9) with each subspace of each
    token quantised asymmetrically (``quantize_rows_asym``) and the weights
    per output channel symmetrically, as in the CoQuant protocol.  With
    x^ = u s_x + z_x and w^ = c_w s_w, each subspace contributes

        sum_k x^_k w^_k = s_x s_w (u . c_w) + z_x s_w (sum_k c_w)

    so Y = sum over the two subspaces of s_x s_w^T (.) (U C_w^T)
    + z_x (s_w (.) colsum(C_w))^T, in fp64.
    """
    xrot = np.asarray(xrot, dtype=np.float32)
    wrot = np.asarray(wrot, dtype=np.float32)
    d = xrot.shape[1]
    if not 0 <= d_hi <= d:
        raise ValueError("d_hi out of range")
    if rows is not None:
        xrot = xrot[np.asarray(rows)]
    if cols is not None:
        wrot = wrot[:, np.asarray(cols)]
    dl = d - d_hi
    out = {}
    y = np.zeros((xrot.shape[0], wrot.shape[1]), dtype=np.float64)
    for tag, xs, ws, bits in (("l", xrot[:, :dl], wrot[:dl], bits_lo), ("h", xrot[:, dl:], wrot[dl:], bits_hi)):
        u, s_x, z_x = quantize_rows_asym(xs, bits)
        cw, s_w = quantize_weight(ws, bits)
        acc = int_matmul(u, cw)
        colsum = cw.astype(np.int64).sum(axis=1)
        sw = s_w.astype(np.float64)
        y = y + (s_x.astype(np.float64)[:, None] * sw[None, :]) * acc.astype(np.float64)
        y = y + z_x.astype(np.float64)[:, None] * (sw * colsum.astype(np.float64))[None, :]
        out.update({f"codes_x{tag}": u, f"s_x{tag}": s_x, f"z_x{tag}": z_x, f"codes_w{tag}": cw, f"s_w{tag}": s_w,
                    f"colsum_{tag}": colsum, f"acc_{tag}": acc})
    out["Y"] = y
    return out


def tq_linear_asym_ref(x, r, l1=None, l2=None, rows=None, cols=None):
    """The rank-augmented layer with per-token asymmetric 4-bit activations:

        Y = s_x s_w^T (.) (U C_w^T) + z_x (s_w (.) colsum(C_w))^T + (X L1) L2      (fp64)

    U, s_x, z_x from ``quantize_rows_asym`` (4 bits), C_w, s_w per output
    channel as in ``tq_linear_ref``; the low-rank branch from the unquantised
    activations as there.
    """
    x = np.asarray(x, dtype=np.float32)
    r = np.asarray(r, dtype=np.float32)
    if rows is not None:
        x = x[np.asarray(rows)]
    if cols is not None:
        r = r[:, np.asarray(cols)]
        if l2 is not None:
            l2 = np.asarray(l2)[:, np.asarray(cols)]
    u, s_x, z_x = quantize_rows_asym(x, 4)
    cw, s_w = quantize_weight(r, 4)
    acc = int_matmul(u, cw)
    colsum = cw.astype(np.int64).sum(axis=1)
    sw = s_w.astype(np.float64)
    y = (s_x.astype(np.float64)[:, None] * sw[None, :]) * acc.astype(np.float64)
    y = y + z_x.astype(np.float64)[:, None] * (sw * colsum.astype(np.float64))[None, :]
    t = None
    if l1 is not None and np.asarray(l1).shape[1] > 0:
        t, ylr = lowrank_branch(x, l1, l2)
        y = y + ylr
    return {"codes_x": u, "s_x": s_x, "z_x": z_x, "codes_w": cw, "s_w": s_w, "colsum": colsum, "acc": acc, "T": t,
            "Y": y}


def hadamard(k: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order k (a power of two), entries +-1."""
    if k < 1 or k & (k - 1):
        raise ValueError("order must be a power of two")
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < k:
        h = np.vstack([np.hstack([h, h]), np.hstack([h, -h])])
    return h


def block_rotation(signs, block: int, perm=None) -> np.ndarray:
    """Dense U = diag(signs) . blockdiag(H_block)/sqrt(block) . P (orthogonal).

    A randomised block-Hadamard basis (CoQuant, rotation paragraph after
    Eq. 3; the randomised Hadamard transforms of "Quantizing With Randomized
    Hadamard Transforms: Efficient Heuristic Now Proven"); P moves column
    perm[j] of the rotated basis to position j.
    """
    signs = np.asarray(signs, dtype=np.float64)
    d = signs.shape[0]
    if d % block:
        raise ValueError("d must be a multiple of the block")
    h = hadamard(block).astype(np.float64) / math.sqrt(block)
    b = np.zeros((d, d), dtype=np.float64)
    for i in range(0, d, block):
        b[i:i + block, i:i + block] = h
    u = signs[:, None] * b
    if perm is not None:
        u = u[:, np.asarray(perm)]
    return u


def rht_rows(x, signs, perm, block: int = 128):
    """The rotation X' = X U of ``block_rotation(signs, block, perm)`` evaluated
    online in fp32, as the fused quantiser does it (the randomised Hadamard
    transform of "Quantizing With Randomized Hadamard Transforms: Efficient
    Heuristic Now Proven", in the block form of the CoQuant rotation after
    Eq. 3):

      v = x * signs                                  (exact: signs are +-1)
      for h = 1, 2, 4, ..., block / 2, within every block of ``block`` columns:
          (v[i], v[i + h]) <- (v[i] + v[i + h], v[i] - v[i + h])   for i with bit h clear
      v = v * fl32(1 / sqrt(block))
      X'[:, j] = v[:, perm[j]]

    Every step is one correctly rounded fp32 operation in this order (the
    fast Walsh-Hadamard transform, natural order, spans increasing), so the
    result is a definite fp32 array that the device reproduces bit for bit.
    """
    v = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)[None, :]
    n, d = v.shape
    if d % block or block & (block - 1):
        raise ValueError("d must be a multiple of a power-of-two block")
    v = v.reshape(n, d // block, block).copy()
    h = 1
    while h < block:
        w = v.reshape(n, d // block, block // (2 * h), 2, h)
        a, b = w[:, :, :, 0, :].copy(), w[:, :, :, 1, :].copy()
        w[:, :, :, 0, :] = a + b
        w[:, :, :, 1, :] = a - b
        h *= 2
    v = v.reshape(n, d) * np.float32(1.0 / math.sqrt(block))
    return np.ascontiguousarray(v[:, np.asarray(perm)], dtype=np.float32)


def tq_linear_mp_rht_ref(x, signs, perm, wrot, d_hi: int, block: int = 128, rows=None, cols=None):
    """Two-subspace output (CoQuant Eq. 9) on unrotated X: the rotation of
    ``rht_rows`` in fp32, then ``tq_linear_mp_ref`` on X' (W' = U^T W is
    rotated offline and given)."""
    x = np.asarray(x, dtype=np.float32)
    if rows is not None:
        x = x[np.asarray(rows)]
    return tq_linear_mp_ref(rht_rows(x, signs, perm, block), wrot, d_hi, cols=cols)


def rotate(x, w, u):
    """Rotation invariance (CoQuant Eq. 3): returns (X U, U^T W), fp64."""
    u = np.asarray(u, dtype=np.float64)
    return np.asarray(x, dtype=np.float64) @ u, u.T @ np.asarray(w, dtype=np.float64)


def subspace_split(x, w, u, d_hi: int):
    """Subspace projections (CoQuant Eq. 4, 6, 7), U = [U_l, U_h], U_h the last d_hi columns.

    Returns X_l = X U_l, X_h = X U_h, W_l = U_l^T W, W_h = U_h^T W (fp64).
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[1]
    ul, uh = u[:, : d - d_hi], u[:, d - d_hi:]
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ ul, x @ uh, ul.T @ w, uh.T @ w

"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

Every mutant replaces one oracle function (via monkeypatch, on the CPU) with a
copy that has one realistic bug: a different operation order, rounding mode,
range, granularity, index, sign, dropped term or transposed operand.  The
test passes when at least one pin of ``test_oracle_pins`` fails under it.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle.tq_oracle as tqo
import test_oracle_pins as pins

_orig = {name: getattr(tqo, name) for name in (
    "quantize_rows", "quantize_weight", "pack_int4", "unpack_int4", "int_matmul",
    "lowrank_branch", "tq_linear_ref", "tq_linear_mp_ref", "hadamard", "block_rotation",
    "subspace_split", "tq_linear_group_ref", "rht_rows", "requantize_lowrank", "tq_linear_qlr_ref", "quantize_rows_asym", "tq_linear_mp_asym_ref", "tq_linear_asym_ref")}


def _q_reciprocal(a, bits=4):
    a = np.asarray(a, dtype=np.float32)
    qmax = (1 << (bits - 1)) - 1
    amax = np.max(np.abs(a), axis=1)
    s = (amax / np.float32(qmax)).astype(np.float32)
    c = np.zeros(a.shape, np.int16)
    live = s > 0
    mult = (np.float32(qmax) / amax[live]).astype(np.float32)
    c[live] = np.clip(np.rint(a[live] * mult[:, None]), -(qmax + 1), qmax)
    return c, s


def _q_half_away(a, bits=4):
    a = np.asarray(a, dtype=np.float32)
    c, s = _orig["quantize_rows"](a, bits)
    qmax = (1 << (bits - 1)) - 1
    live = s > 0
    q = (a[live] / s[live][:, None]).astype(np.float32)
    c[live] = np.clip(np.sign(q) * np.floor(np.abs(q) + 0.5), -(qmax + 1), qmax)
    return c, s


def _q_qmax_pow2(a, bits=4):
    return _q_scale_by(a, bits, 1 << (bits - 1))  # q_max taken as 2^(N-1)


def _q_scale_by(a, bits, qmax_used):
    a = np.asarray(a, dtype=np.float32)
    qmax = (1 << (bits - 1)) - 1
    amax = np.max(np.abs(a), axis=1)
    s = (amax / np.float32(qmax_used)).astype(np.float32)
    c = np.zeros(a.shape, np.int16)
    live = s > 0
    c[live] = np.clip(np.rint((a[live] / s[live][:, None]).astype(np.float32)), -(qmax + 1), qmax)
    return c, s


def _q_per_tensor(a, bits=4):
    a = np.asarray(a, dtype=np.float32)
    qmax = (1 << (bits - 1)) - 1
    amax = np.float32(np.max(np.abs(a))) if a.size else np.float32(0)
    s = np.full(a.shape[0], amax / np.float32(qmax), dtype=np.float32)
    c = np.zeros(a.shape, np.int16)
    if amax > 0:
        c = np.clip(np.rint((a / s[:, None]).astype(np.float32)), -(qmax + 1), qmax).astype(np.int16)
    return c, s


def _q_no_clamp_low(a, bits=4):
    a = np.asarray(a, dtype=np.float32)
    qmax = (1 << (bits - 1)) - 1
    c, s = _orig["quantize_rows"](a, bits)
    live = s > 0
    c[live] = np.clip(np.rint((a[live] / s[live][:, None]).astype(np.float32)), -qmax, qmax)
    return c, s


def _w_per_input_channel(w, bits=4):
    c, s = tqo.quantize_rows(np.asarray(w, np.float32), bits)  # rows of W instead of columns
    return np.ascontiguousarray(c.T), s


def _pack_swapped(codes):
    c = np.asarray(codes)
    u = (c.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[..., 1::2] | (u[..., 0::2] << 4)).astype(np.uint8)


def _unpack_no_sign(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int16)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _matmul_drop_last(cx, cw):
    cx, cw = np.asarray(cx), np.asarray(cw)
    return _orig["int_matmul"](cx[:, :-1], cw[:, :-1])  # last k term dropped


def _matmul_int16_wrap(cx, cw):
    return _orig["int_matmul"](cx, cw).astype(np.int16).astype(np.int64)


def _lowrank_quantized_x(x, l1, l2):
    c, s = tqo.quantize_rows(x, 4)
    return _orig["lowrank_branch"](c * s[:, None].astype(np.float64), l1, l2)


def _lowrank_sign(x, l1, l2):
    t, y = _orig["lowrank_branch"](x, l1, l2)
    return t, -y


def _lowrank_drop(x, l1, l2):
    t, y = _orig["lowrank_branch"](x, l1, l2)
    return t, 0 * y


def _linear_sx_only_first(x, r, l1=None, l2=None, rows=None, cols=None, bits=4):
    out = _orig["tq_linear_ref"](x, r, l1, l2, rows, cols, bits)
    # every row dequantised with the first token's scale
    base = out["s_x"][0] * out["s_w"].astype(np.float64)[None, :] * out["acc"]
    true = out["s_x"].astype(np.float64)[:, None] * out["s_w"].astype(np.float64)[None, :] * out["acc"]
    out["Y"] = out["Y"] - true + base
    return out


def _mp_bits_swapped(xrot, wrot, d_hi, rows=None, cols=None, bits_lo=4, bits_hi=8):
    return _orig["tq_linear_mp_ref"](xrot, wrot, d_hi, rows, cols, bits_hi, bits_lo)


def _mp_shared_scale(xrot, wrot, d_hi, rows=None, cols=None, bits_lo=4, bits_hi=8):
    out = _orig["tq_linear_mp_ref"](xrot, wrot, d_hi, rows, cols, bits_lo, bits_hi)
    y = out["s_xl"][:, None].astype(np.float64) * out["s_wl"][None, :] * (out["acc_l"] + out["acc_h"])
    out["Y"] = y
    return out


def _mp_hi_first(xrot, wrot, d_hi, rows=None, cols=None, bits_lo=4, bits_hi=8):
    x = np.asarray(xrot, np.float32)
    w = np.asarray(wrot, np.float32)
    d = x.shape[1]
    order = np.r_[d_hi:d, 0:d_hi]  # the FIRST d_hi coordinates used as the high subspace
    return _orig["tq_linear_mp_ref"](x[:, order], w[order], d_hi, rows, cols, bits_lo, bits_hi)


def _hadamard_bad(k):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < k:
        h = np.vstack([np.hstack([h, h]), np.hstack([-h, h])])
    return h


def _rotation_no_norm(signs, block, perm=None):
    return _orig["block_rotation"](signs, block, perm) * np.sqrt(1.0 + 1.0 / block)


def _split_swapped(x, w, u, d_hi):
    u = np.asarray(u, dtype=np.float64)
    uh, ul = u[:, :d_hi], u[:, d_hi:]
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    return x @ ul, x @ uh, ul.T @ w, uh.T @ w


def _group_first_l2(x, rs, l1s=None, l2s=None, rows=None, bits=4):
    # every layer's low-rank product taken with its own L1 but L2 columns of
    # the first layer cut or padded to its width
    l2x = [np.resize(l2s[0], l2.shape).astype(np.float32) for l2 in l2s]
    return _orig["tq_linear_group_ref"](x, rs, l1s, l2x, rows, bits)


def _group_reversed(x, rs, l1s=None, l2s=None, rows=None, bits=4):
    out = _orig["tq_linear_group_ref"](x, rs[::-1], l1s[::-1], l2s[::-1], rows, bits)
    out["layers"] = out["layers"][::-1]
    return out


def _group_l1_shared(x, rs, l1s=None, l2s=None, rows=None, bits=4):
    return _orig["tq_linear_group_ref"](x, rs, [l1s[0]] * len(l1s), l2s, rows, bits)


def _rht_sub_swapped(x, signs, perm, block=128):
    # butterfly difference taken the other way round: (v[i + h] - v[i])
    return _rht_generic(x, signs, perm, block, flip=True)


def _rht_generic(x, signs, perm, block=128, flip=False, inverse_perm=False, scale=None, signs_after=False):
    v = np.asarray(x, dtype=np.float32)
    if not signs_after:
        v = v * np.asarray(signs, dtype=np.float32)[None, :]
    n, d = v.shape
    v = v.reshape(n, d // block, block).copy()
    h = 1
    while h < block:
        w = v.reshape(n, d // block, block // (2 * h), 2, h)
        a, b = w[:, :, :, 0, :].copy(), w[:, :, :, 1, :].copy()
        w[:, :, :, 0, :] = a + b
        w[:, :, :, 1, :] = (b - a) if flip else (a - b)
        h *= 2
    v = v.reshape(n, d) * np.float32(scale if scale is not None else 1.0 / np.sqrt(block))
    if signs_after:
        v = v * np.asarray(signs, dtype=np.float32)[None, :]
    p = np.asarray(perm)
    if inverse_perm:
        p = np.argsort(p)
    return np.ascontiguousarray(v[:, p], dtype=np.float32)


def _rht_inverse_perm(x, signs, perm, block=128):
    return _rht_generic(x, signs, perm, block, inverse_perm=True)


def _rht_scale_by_block(x, signs, perm, block=128):
    return _rht_generic(x, signs, perm, block, scale=1.0 / block)


def _rht_signs_after(x, signs, perm, block=128):
    return _rht_generic(x, signs, perm, block, signs_after=True)


def _requant_no_su(acc1, s_u, bits=4):  # the column scales of U left out of the first stage
    return _orig["requantize_lowrank"](acc1, np.ones_like(np.asarray(s_u, np.float32)), bits)


def _requant_per_column(acc1, s_u, bits=4):  # re-quantised per rank column instead of per token
    t = (np.asarray(acc1).astype(np.float32) * np.asarray(s_u, np.float32)[None, :]).astype(np.float32)
    c, s = _orig["quantize_rows"](t.T, bits)
    return t, c.T, s


def _requant_trunc(acc1, s_u, bits=4):  # codes truncated toward zero
    t, c, s = _orig["requantize_lowrank"](acc1, s_u, bits)
    live = s > 0
    c[live] = np.clip(np.trunc((t[live] / s[live][:, None]).astype(np.float32)), -8, 7)
    return t, c, s


def _requant_8bit(acc1, s_u, bits=4):  # the intermediate kept at 8 bits
    return _orig["requantize_lowrank"](acc1, s_u, 8)


def _qlr_generic(x, r, u, v, rows=None, cols=None, bits=4, lr_sx=True, lr_st=True, unrequantised=False):
    out = _orig["tq_linear_qlr_ref"](x, r, u, v, rows, cols, bits)
    xs = np.asarray(x) if rows is None else np.asarray(x)[np.asarray(rows)]
    rs = np.asarray(r) if cols is None else np.asarray(r)[:, np.asarray(cols)]
    y0 = _orig["tq_linear_ref"](xs, rs, bits=bits)["Y"]
    sx = out["s_x"].astype(np.float64)[:, None] if lr_sx else 1.0
    st = out["s_t"].astype(np.float64)[:, None] if lr_st else 1.0
    tt = out["codes_t"].astype(np.float64) * st
    if unrequantised:
        tt = out["t"].astype(np.float64)
    vv = out["codes_v"].astype(np.float64) * out["s_v"].astype(np.float64)[:, None]
    out["Y"] = y0 + sx * (tt @ vv.T)
    return out


def _qlr_lr_no_sx(x, r, u, v, rows=None, cols=None, bits=4):  # the token scale missing from the low-rank term
    return _qlr_generic(x, r, u, v, rows, cols, bits, lr_sx=False)


def _qlr_lr_no_st(x, r, u, v, rows=None, cols=None, bits=4):  # the stage scale missing
    return _qlr_generic(x, r, u, v, rows, cols, bits, lr_st=False)


def _qlr_unrequantised(x, r, u, v, rows=None, cols=None, bits=4):  # the fp32 first stage fed on, not its codes
    return _qlr_generic(x, r, u, v, rows, cols, bits, unrequantised=True)


def _asym_generic(a, bits=4, qm_used=None, clip_lo=0, clip_hi=None, z_from="min", sub_after=False):
    a = np.asarray(a, dtype=np.float32)
    qm = (1 << bits) - 1
    qmu = qm if qm_used is None else qm_used
    hi = qm if clip_hi is None else clip_hi
    mn, mx = a.min(axis=1), a.max(axis=1)
    z = mn if z_from == "min" else (mx if z_from == "max" else np.zeros_like(mn))
    s = ((mx - mn).astype(np.float32) / np.float32(qmu)).astype(np.float32)
    u = np.zeros(a.shape, np.int16)
    live = s > 0
    if sub_after:  # x / s - z / s instead of (x - z) / s
        q = (a[live] / s[live][:, None]).astype(np.float32) - (z[live] / s[live]).astype(np.float32)[:, None]
    else:
        q = ((a[live] - z[live][:, None]).astype(np.float32) / s[live][:, None]).astype(np.float32)
    u[live] = np.clip(np.rint(q), clip_lo, hi)
    return u, s, z.astype(np.float32)


def _asym_qmax_signed(a, bits=4):  # the symmetric q_max 2^(N-1) - 1 as the step count
    return _asym_generic(a, bits, qm_used=(1 << (bits - 1)) - 1)


def _asym_signed_clip(a, bits=4):  # codes clipped to the signed range
    return _asym_generic(a, bits, clip_lo=-(1 << (bits - 1)), clip_hi=(1 << (bits - 1)) - 1)


def _asym_z_max(a, bits=4):  # zero-point at the maximum
    return _asym_generic(a, bits, z_from="max")


def _asym_sub_after(a, bits=4):  # the zero-point subtracted after the division
    return _asym_generic(a, bits, sub_after=True)


def _mp_asym_no_zero_term(xrot, wrot, d_hi, rows=None, cols=None, bits_lo=4, bits_hi=8):  # z s_w colsum dropped
    out = _orig["tq_linear_mp_asym_ref"](xrot, wrot, d_hi, rows, cols, bits_lo, bits_hi)
    y = 0.0
    for t in ("l", "h"):
        y = y + (out[f"s_x{t}"].astype(np.float64)[:, None] * out[f"s_w{t}"].astype(np.float64)[None, :]) * \
            out[f"acc_{t}"].astype(np.float64)
    out["Y"] = y
    return out


def _mp_asym_shared_z(xrot, wrot, d_hi, rows=None, cols=None, bits_lo=4, bits_hi=8):  # the 4-bit z used for both
    out = _orig["tq_linear_mp_asym_ref"](xrot, wrot, d_hi, rows, cols, bits_lo, bits_hi)
    y = 0.0
    for t in ("l", "h"):
        sw = out[f"s_w{t}"].astype(np.float64)
        y = y + (out[f"s_x{t}"].astype(np.float64)[:, None] * sw[None, :]) * out[f"acc_{t}"].astype(np.float64)
        y = y + out["z_xl"].astype(np.float64)[:, None] * (sw * out[f"colsum_{t}"].astype(np.float64))[None, :]
    out["Y"] = y
    return out


def _linear_asym_no_zero_term(x, r, l1=None, l2=None, rows=None, cols=None):  # z s_w colsum dropped
    out = _orig["tq_linear_asym_ref"](x, r, l1, l2, rows, cols)
    y = (out["s_x"].astype(np.float64)[:, None] * out["s_w"].astype(np.float64)[None, :]) * out["acc"]
    if out["T"] is not None:
        y = y + out["T"] @ np.asarray(l2 if cols is None else np.asarray(l2)[:, cols], np.float64)
    out["Y"] = y
    return out


def _linear_asym_offset_codes(x, r, l1=None, l2=None, rows=None, cols=None):  # codes u - 8 without the 8 s term
    out = _orig["tq_linear_asym_ref"](x, r, l1, l2, rows, cols)
    sw = out["s_w"].astype(np.float64)
    y = (out["s_x"].astype(np.float64)[:, None] * sw[None, :]) * _orig["int_matmul"](out["codes_x"] - 8, out["codes_w"])
    y = y + out["z_x"].astype(np.float64)[:, None] * (sw * out["colsum"])[None, :]
    if out["T"] is not None:
        y = y + out["T"] @ np.asarray(l2 if cols is None else np.asarray(l2)[:, cols], np.float64)
    out["Y"] = y
    return out


MUTANTS = {
    "quantize_rows": [_q_reciprocal, _q_half_away, _q_qmax_pow2, _q_per_tensor, _q_no_clamp_low],
    "quantize_weight": [_w_per_input_channel],
    "pack_int4": [_pack_swapped],
    "unpack_int4": [_unpack_no_sign],
    "int_matmul": [_matmul_drop_last, _matmul_int16_wrap],
    "lowrank_branch": [_lowrank_quantized_x, _lowrank_sign, _lowrank_drop],
    "tq_linear_ref": [_linear_sx_only_first],
    "tq_linear_mp_ref": [_mp_bits_swapped, _mp_shared_scale, _mp_hi_first],
    "hadamard": [_hadamard_bad],
    "block_rotation": [_rotation_no_norm],
    "subspace_split": [_split_swapped],
    "tq_linear_group_ref": [_group_first_l2, _group_reversed, _group_l1_shared],
    "rht_rows": [_rht_sub_swapped, _rht_inverse_perm, _rht_scale_by_block, _rht_signs_after],
    "requantize_lowrank": [_requant_no_su, _requant_per_column, _requant_trunc, _requant_8bit],
    "tq_linear_qlr_ref": [_qlr_lr_no_sx, _qlr_lr_no_st, _qlr_unrequantised],
    "quantize_rows_asym": [_asym_qmax_signed, _asym_signed_clip, _asym_z_max, _asym_sub_after],
    "tq_linear_mp_asym_ref": [_mp_asym_no_zero_term, _mp_asym_shared_z],
    "tq_linear_asym_ref": [_linear_asym_no_zero_term, _linear_asym_offset_codes],
}

CASES = [(name, f) for name, fs in MUTANTS.items() for f in fs]


def _run_all_pins():
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception as e:  # noqa: BLE001 -- any failure counts as "caught"
            failed.append((pin.__name__, type(e).__name__))
    # the slow brute force only for quantiser mutants that may slip past the rest
    return failed


@pytest.mark.parametrize("target,mutant", CASES, ids=[f"{n}:{f.__name__}" for n, f in CASES])
def test_mutant_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(tqo, target, mutant)
    failed = _run_all_pins()
    if not failed and target == "quantize_rows":
        try:
            pins.pin_quantizer_bruteforce(amaxes=(3.0,))
        except Exception as e:  # noqa: BLE001
            failed.append(("pin_quantizer_bruteforce", type(e).__name__))
    assert failed, f"mutant {mutant.__name__} of {target} passed every pin"


def test_unmutated_oracle_passes_all_pins():
    assert _run_all_pins() == []

"""Thin Python binding of the C ABI in ``include/tq.h`` (libtq.so).

Argument marshalling only: every computation runs in the HIP library.
PyTorch provides device memory (tensors) and the current stream.  Each
function has the name of the C entry point it calls; outputs that are not
passed in are allocated with ``torch.empty`` / ``torch.zeros``.
"""

from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB

TQ_F32, TQ_BF16 = 0, 1

_STATUS = {
    0: "TQ_OK", -1: "TQ_ERR_NULL", -2: "TQ_ERR_SHAPE", -3: "TQ_ERR_DTYPE", -4: "TQ_ERR_BITS",
    -5: "TQ_ERR_ALIGN", -6: "TQ_ERR_WORKSPACE", -7: "TQ_ERR_HIP",
}

EXPORTS = (
    "tq_status_string", "tq_version", "tq_codes_bytes", "tq_pack_weight", "tq_lowrank_bytes",
    "tq_pack_lowrank", "tq_quantize_act", "tq_linear_workspace_bytes", "tq_linear_workspace_offsets", "tq_linear",
    "tq_linear_mp_workspace_bytes", "tq_linear_mp", "tq_debug_accumulate", "tq_profile_enable",
    "tq_profile_read", "tq_profile_reset", "tq_lowrank_group_bytes", "tq_pack_lowrank_group",
    "tq_linear_group_workspace_bytes", "tq_linear_group", "tq_linear_mp_workspace_offsets", "tq_rht_bytes",
    "tq_pack_rht", "tq_linear_mp_rht", "tq_lowrank_q_bytes", "tq_pack_lowrank_q", "tq_linear_qlr_workspace_bytes",
    "tq_linear_qlr_workspace_offsets", "tq_linear_qlr", "tq_weight_colsum", "tq_linear_mp_asym_workspace_bytes",
    "tq_linear_mp_asym_workspace_offsets", "tq_linear_mp_asym", "tq_linear_mp_bits", "tq_linear_asym_workspace_bytes",
    "tq_linear_asym_workspace_offsets", "tq_linear_asym", "tq_linear_debug", "tq_linear_mp_bits_debug",
    "tq_linear_asym_debug", "tq_linear_mp_asym_debug", "tq_linear_qlr_debug", "tq_linear_noalloc",
    "tq_debug_linear_handoff",
    "tq_debug_stream_read", "tq_debug_mfma_ceiling", "tq_debug_accumulate_i8", "tq_debug_gemm_w4a4",
)

NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024  # TQ_NOALLOC_SCRATCH_BYTES of include/tq.h


class TQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libtq.so (built in-tree by ``python -m rank_augmented_quantized_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB
    if not os.path.exists(path):
        raise ImportError(
            f"HIP library {path} is missing; build it with `python -m rank_augmented_quantized_amd.build`")
    lib = ctypes.CDLL(path)
    i64, ptr, st, c_int, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_size_t
    sigs = {
        "tq_status_string": (ctypes.c_char_p, [c_int]),
        "tq_version": (c_int, []),
        "tq_codes_bytes": (sz, [i64, i64, c_int]),
        "tq_pack_weight": (st, [ptr, c_int, i64, i64, c_int, ptr, ptr, ptr]),
        "tq_lowrank_bytes": (sz, [i64, i64, i64]),
        "tq_pack_lowrank": (st, [ptr, ptr, c_int, i64, i64, i64, ptr, ptr]),
        "tq_quantize_act": (st, [ptr, c_int, i64, i64, c_int, ptr, ptr, ptr]),
        "tq_linear_workspace_bytes": (sz, [i64, i64, i64, i64]),
        "tq_linear": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, c_int, ptr, sz, ptr]),
        "tq_linear_workspace_offsets": (st, [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]),
        "tq_linear_mp_workspace_bytes": (sz, [i64, i64, i64]),
        "tq_linear_mp": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, ptr, c_int, ptr, sz, ptr]),
        "tq_debug_accumulate": (st, [ptr, ptr, i64, i64, i64, c_int, ptr, ptr]),
        "tq_debug_accumulate_i8": (st, [ptr, ptr, i64, i64, i64, ptr, ptr]),
        "tq_debug_gemm_w4a4": (st, [ptr, c_int, ptr, ptr, ptr, i64, i64, i64, ptr, ptr]),
        "tq_profile_enable": (st, [c_int]),
        "tq_profile_read": (c_int, [ctypes.POINTER(KernelStat), c_int]),
        "tq_profile_reset": (st, []),
        "tq_lowrank_group_bytes": (sz, [i64, ptr, i64, i64]),
        "tq_pack_lowrank_group": (st, [ptr, ptr, c_int, i64, ptr, i64, i64, ptr, ptr]),
        "tq_linear_group_workspace_bytes": (sz, [i64, i64, ptr, i64, i64]),
        "tq_linear_group": (st, [ptr, c_int, i64, i64, ptr, i64, i64, ptr, ptr, ptr, ptr, c_int, ptr, sz, ptr]),
        "tq_linear_mp_workspace_offsets": (st, [i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]),
        "tq_rht_bytes": (sz, [i64]),
        "tq_pack_rht": (st, [ptr, ptr, i64, ptr, ptr]),
        "tq_linear_mp_rht": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, ptr, ptr, c_int, ptr, sz,
                                  ptr]),
        "tq_lowrank_q_bytes": (sz, [i64, i64, i64]),
        "tq_pack_lowrank_q": (st, [ptr, ptr, c_int, i64, i64, i64, ptr, ptr]),
        "tq_linear_qlr_workspace_bytes": (sz, [i64, i64, i64]),
        "tq_linear_qlr_workspace_offsets": (st, [i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]),
        "tq_linear_qlr": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, c_int, ptr, sz, ptr]),
        "tq_weight_colsum": (st, [ptr, i64, i64, c_int, ptr, ptr]),
        "tq_linear_asym_workspace_bytes": (sz, [i64, i64, i64, i64]),
        "tq_linear_asym_workspace_offsets": (st, [i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]),
        "tq_linear_asym": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, ptr, c_int, ptr, sz, ptr]),
        "tq_linear_mp_bits": (st, [ptr, c_int, i64, i64, i64, i64, c_int, c_int, ptr, ptr, ptr, ptr, ptr, c_int, ptr,
                                   sz, ptr]),
        "tq_linear_mp_asym_workspace_bytes": (sz, [i64, i64, i64]),
        "tq_linear_mp_asym_workspace_offsets": (st, [i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]),
        "tq_linear_mp_asym": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, ptr, ptr, ptr, c_int, ptr,
                                   sz, ptr]),
        "tq_linear_debug": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, c_int, ptr, sz, ptr, ptr]),
        "tq_linear_mp_bits_debug": (st, [ptr, c_int, i64, i64, i64, i64, c_int, c_int, ptr, ptr, ptr, ptr, ptr,
                                         c_int, ptr, sz, ptr, ptr, ptr]),
        "tq_linear_asym_debug": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, ptr, c_int, ptr, sz, ptr,
                                      ptr]),
        "tq_linear_mp_asym_debug": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, ptr, ptr, ptr, c_int,
                                         ptr, sz, ptr, ptr, ptr]),
        "tq_linear_qlr_debug": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, c_int, ptr, sz, ptr, ptr,
                                     ptr]),
        "tq_linear_noalloc": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, c_int, ptr]),
        "tq_debug_linear_handoff": (st, [ptr, c_int, i64, i64, i64, i64, ptr, ptr, ptr, ptr, c_int, ptr, sz,
                                         ctypes.c_uint, c_int, ptr]),
        "tq_debug_stream_read": (st, [ptr, sz, ptr, c_int, ptr]),
        "tq_debug_mfma_ceiling": (st, [c_int, c_int, ptr, ptr]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise TQError(fn, status)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t) -> int:
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def tq_codes_bytes(rows: int, k: int, bits: int) -> int:
    return load().tq_codes_bytes(rows, k, bits)


def tq_pack_weight(W, bits: int = 4, w_codes=None, s_w=None):
    """Per-output-channel quantisation of a d x m weight -> (codes m x d*bits/8 uint8, s_w fp32 m)."""
    lib = load()
    _need_cuda(W)
    d, m = W.shape
    if w_codes is None:
        w_codes = torch.empty((m, d * (4 if bits <= 4 else 8) // 8), dtype=torch.uint8, device=W.device)
    if s_w is None:
        s_w = torch.empty(m, dtype=torch.float32, device=W.device)
    _check("tq_pack_weight", lib.tq_pack_weight(_p(W), _dt(W), d, m, bits, _p(w_codes), _p(s_w), _stream(W)))
    return w_codes, s_w


def tq_pack_lowrank(L1, L2, out=None):
    """Lay out the low-rank factors (L1 d x r, L2 r x m) for tq_linear."""
    lib = load()
    _need_cuda(L1, L2)
    d, r = L1.shape
    m = L2.shape[1]
    if out is None:
        out = torch.empty(lib.tq_lowrank_bytes(d, m, r), dtype=torch.uint8, device=L1.device)
    _check("tq_pack_lowrank", lib.tq_pack_lowrank(_p(L1), _p(L2), _dt(L1), d, m, r, _p(out), _stream(L1)))
    return out


def tq_quantize_act(X, bits: int = 4, x_codes=None, s_x=None):
    """Per-token quantisation of n x d activations -> (codes n x d*bits/8 uint8, s_x fp32 n)."""
    lib = load()
    _need_cuda(X)
    n, d = X.shape
    if x_codes is None:
        x_codes = torch.empty((n, d * bits // 8), dtype=torch.uint8, device=X.device)
    if s_x is None:
        s_x = torch.empty(n, dtype=torch.float32, device=X.device)
    _check("tq_quantize_act", lib.tq_quantize_act(_p(X), _dt(X), n, d, bits, _p(x_codes), _p(s_x), _stream(X)))
    return x_codes, s_x


def tq_linear_workspace_bytes(n: int, d: int, m: int, r: int) -> int:
    return load().tq_linear_workspace_bytes(n, d, m, r)


def tq_linear_workspace_offsets(n: int, d: int, m: int, r: int) -> dict:
    """Byte offsets of s_x, the activation codes, T and the hand-off words inside tq_linear's workspace."""
    off = (ctypes.c_size_t * 4)()
    _check("tq_linear_workspace_offsets", load().tq_linear_workspace_offsets(n, d, m, r, off))
    return {"s_x": off[0], "x_codes": off[1], "T": off[2], "sync": off[3]}


def linear_workspace(n: int, d: int, m: int, r: int, device) -> torch.Tensor:
    """A zero-filled workspace for tq_linear (its counter block must start at zero)."""
    return torch.zeros(max(1, tq_linear_workspace_bytes(n, d, m, r)), dtype=torch.uint8, device=device)


def tq_linear(X, w_codes, s_w, lowrank, m: int, r: int, y_dtype=torch.bfloat16, Y=None, ws=None, acc=None):
    """Y = s_x s_w (Q4(X) Q4(R)) + (X L1) L2 for X n x d.  acc (n x m int32, optional): the kernels' exact
    residual sums, through tq_linear_debug."""
    lib = load()
    _need_cuda(X, w_codes, s_w, lowrank, Y, ws, acc)
    n, d = X.shape
    if Y is None:
        Y = torch.empty((n, m), dtype=y_dtype, device=X.device)
    if ws is None:
        ws = linear_workspace(n, d, m, r, X.device)
    if acc is None:
        _check("tq_linear", lib.tq_linear(_p(X), _dt(X), n, d, m, r, _p(w_codes), _p(s_w), _p(lowrank),
                                          _p(Y), _dt(Y), _p(ws), ws.numel(), _stream(X)))
    else:
        _check("tq_linear_debug", lib.tq_linear_debug(_p(X), _dt(X), n, d, m, r, _p(w_codes), _p(s_w), _p(lowrank),
                                                      _p(Y), _dt(Y), _p(ws), ws.numel(), _p(acc), _stream(X)))
    return Y


def tq_linear_noalloc(X, w_codes, s_w, lowrank, m: int, r: int, Y):
    """tq_linear with the library's own device scratch instead of a workspace (no allocation: Y is passed in)."""
    lib = load()
    _need_cuda(X, w_codes, s_w, lowrank, Y)
    n, d = X.shape
    _check("tq_linear_noalloc", lib.tq_linear_noalloc(_p(X), _dt(X), n, d, m, r, _p(w_codes), _p(s_w), _p(lowrank),
                                                      _p(Y), _dt(Y), _stream(X)))
    return Y


def tq_debug_linear_handoff(X, w_codes, s_w, lowrank, m: int, r: int, Y, ws, spin: int, silent: bool):
    """tq_linear with the one-launch path's waits limited to ``spin`` polls (and, if ``silent``, never satisfied)."""
    lib = load()
    _need_cuda(X, w_codes, s_w, lowrank, Y, ws)
    n, d = X.shape
    _check("tq_debug_linear_handoff", lib.tq_debug_linear_handoff(
        _p(X), _dt(X), n, d, m, r, _p(w_codes), _p(s_w), _p(lowrank), _p(Y), _dt(Y), _p(ws), ws.numel(), spin,
        1 if silent else 0, _stream(X)))
    return Y


def tq_debug_stream_read(buf, out, blocks: int):
    """Read all of ``buf`` (a CUDA tensor, whole number of 16-byte units) once with the decode kernel's loads;
    ``out``: an int32 CUDA tensor of at least ``blocks`` elements (one XOR per block)."""
    lib = load()
    _need_cuda(buf, out)
    nbytes = buf.numel() * buf.element_size()
    if out.numel() < blocks:
        raise ValueError("out holds fewer words than blocks")
    _check("tq_debug_stream_read", lib.tq_debug_stream_read(_p(buf), nbytes, _p(out), blocks, _stream(buf)))
    return out


def tq_debug_mfma_ceiling(out, iters: int, blocks: int):
    """Chain ``iters`` rounds of 8 int8 32x32x32 MFMAs per wave in ``blocks`` blocks of 512 threads;
    ``out``: an int32 CUDA tensor of at least 512 ``blocks`` elements (one sum per thread)."""
    lib = load()
    _need_cuda(out)
    if out.numel() < 512 * blocks:
        raise ValueError("out holds fewer words than 512 x blocks")
    _check("tq_debug_mfma_ceiling", lib.tq_debug_mfma_ceiling(iters, blocks, _p(out), _stream(out)))
    return out


def tq_linear_mp_workspace_bytes(n: int, d: int, d_hi: int) -> int:
    return load().tq_linear_mp_workspace_bytes(n, d, d_hi)


def tq_linear_mp(Xrot, d_hi: int, wl_codes, s_wl, wh_codes, s_wh, m: int, y_dtype=torch.bfloat16, Y=None, ws=None,
                 bits=(4, 8), acc_l=None, acc_h=None):
    """Y = Q4(X_l) Q4(W_l) + Q8(X_h) Q8(W_h), X_h = the last d_hi columns of Xrot (bits=(3, 6): Q3 and Q6).
    acc_l / acc_h (n x m int32, optional): the kernel's exact sums of both subspaces, through
    tq_linear_mp_bits_debug."""
    lib = load()
    _need_cuda(Xrot, wl_codes, s_wl, wh_codes, s_wh, Y, ws, acc_l, acc_h)
    n, d = Xrot.shape
    if Y is None:
        Y = torch.empty((n, m), dtype=y_dtype, device=Xrot.device)
    if ws is None:
        ws = torch.empty(max(1, tq_linear_mp_workspace_bytes(n, d, d_hi)), dtype=torch.uint8, device=Xrot.device)
    if acc_l is not None:
        _check("tq_linear_mp_bits_debug", lib.tq_linear_mp_bits_debug(
            _p(Xrot), _dt(Xrot), n, d, m, d_hi, bits[0], bits[1], _p(wl_codes), _p(s_wl), _p(wh_codes), _p(s_wh),
            _p(Y), _dt(Y), _p(ws), ws.numel(), _p(acc_l), _p(acc_h), _stream(Xrot)))
    elif tuple(bits) == (4, 8):
        _check("tq_linear_mp", lib.tq_linear_mp(_p(Xrot), _dt(Xrot), n, d, m, d_hi, _p(wl_codes), _p(s_wl),
                                                _p(wh_codes), _p(s_wh), _p(Y), _dt(Y), _p(ws), ws.numel(),
                                                _stream(Xrot)))
    else:
        _check("tq_linear_mp_bits", lib.tq_linear_mp_bits(_p(Xrot), _dt(Xrot), n, d, m, d_hi, bits[0], bits[1],
                                                          _p(wl_codes), _p(s_wl), _p(wh_codes), _p(s_wh), _p(Y),
                                                          _dt(Y), _p(ws), ws.numel(), _stream(Xrot)))
    return Y


def _i64s(ms):
    return (ctypes.c_int64 * len(ms))(*[int(v) for v in ms])


def tq_lowrank_group_bytes(d: int, ms, r: int) -> int:
    return load().tq_lowrank_group_bytes(d, _i64s(ms), len(ms), r)


def tq_pack_lowrank_group(L1s, L2s, out=None):
    """Lay out G layers' low-rank factors (L1s[g] d x r, L2s[g] r x m[g]) for tq_linear_group."""
    lib = load()
    _need_cuda(*L1s, *L2s)
    d, r = L1s[0].shape
    ms = [L2.shape[1] for L2 in L2s]
    if out is None:
        out = torch.empty(max(1, tq_lowrank_group_bytes(d, ms, r)), dtype=torch.uint8, device=L1s[0].device)
    p1 = (ctypes.c_void_p * len(L1s))(*[t.data_ptr() for t in L1s])
    p2 = (ctypes.c_void_p * len(L2s))(*[t.data_ptr() for t in L2s])
    _check("tq_pack_lowrank_group", lib.tq_pack_lowrank_group(p1, p2, _dt(L1s[0]), d, _i64s(ms), len(ms), r,
                                                              _p(out), _stream(L1s[0])))
    return out


def tq_linear_group_workspace_bytes(n: int, d: int, ms, r: int) -> int:
    return load().tq_linear_group_workspace_bytes(n, d, _i64s(ms), len(ms), r)


def linear_group_workspace(n: int, d: int, ms, r: int, device) -> torch.Tensor:
    """A zero-filled workspace for tq_linear_group."""
    return torch.zeros(max(1, tq_linear_group_workspace_bytes(n, d, ms, r)), dtype=torch.uint8, device=device)


def tq_linear_group(X, w_codes, s_w, lowrank, ms, r: int, y_dtype=torch.bfloat16, Y=None, ws=None):
    """G layers sharing X: w_codes / s_w stacked in channel order (ms[g] channels each); Y n x sum(ms)."""
    lib = load()
    _need_cuda(X, w_codes, s_w, lowrank, Y, ws)
    n, d = X.shape
    mt = int(sum(ms))
    if Y is None:
        Y = torch.empty((n, mt), dtype=y_dtype, device=X.device)
    if ws is None:
        ws = linear_group_workspace(n, d, ms, r, X.device)
    _check("tq_linear_group", lib.tq_linear_group(_p(X), _dt(X), n, d, _i64s(ms), len(ms), r, _p(w_codes),
                                                  _p(s_w), _p(lowrank), _p(Y), _dt(Y), _p(ws), ws.numel(),
                                                  _stream(X)))
    return Y


def tq_linear_mp_workspace_offsets(n: int, d: int, d_hi: int) -> dict:
    """Byte offsets of the two subspaces' scales and codes inside tq_linear_mp's workspace."""
    off = (ctypes.c_size_t * 4)()
    _check("tq_linear_mp_workspace_offsets", load().tq_linear_mp_workspace_offsets(n, d, d_hi, off))
    return {"s_xl": off[0], "s_xh": off[1], "x_codes_l": off[2], "x_codes_h": off[3]}


def tq_pack_rht(signs, perm, out=None):
    """Lay out a rotation (signs fp32 +-1, perm int32, both of length d) for tq_linear_mp_rht."""
    lib = load()
    _need_cuda(signs, perm)
    d = signs.shape[0]
    if out is None:
        out = torch.empty(max(1, lib.tq_rht_bytes(d)), dtype=torch.uint8, device=signs.device)
    _check("tq_pack_rht", lib.tq_pack_rht(_p(signs), _p(perm), d, _p(out), _stream(signs)))
    return out


def tq_linear_mp_rht(X, d_hi: int, rot, wl_codes, s_wl, wh_codes, s_wh, m: int, y_dtype=torch.bfloat16, Y=None,
                     ws=None):
    """tq_linear_mp on unrotated X, the rotation (tq_pack_rht) applied inside the quantiser."""
    lib = load()
    _need_cuda(X, rot, wl_codes, s_wl, wh_codes, s_wh, Y, ws)
    n, d = X.shape
    if Y is None:
        Y = torch.empty((n, m), dtype=y_dtype, device=X.device)
    if ws is None:
        ws = torch.empty(max(1, tq_linear_mp_workspace_bytes(n, d, d_hi)), dtype=torch.uint8, device=X.device)
    _check("tq_linear_mp_rht", lib.tq_linear_mp_rht(_p(X), _dt(X), n, d, m, d_hi, _p(rot), _p(wl_codes), _p(s_wl),
                                                    _p(wh_codes), _p(s_wh), _p(Y), _dt(Y), _p(ws), ws.numel(),
                                                    _stream(X)))
    return Y


def tq_lowrank_q_bytes(d: int, m: int, r: int) -> int:
    return load().tq_lowrank_q_bytes(d, m, r)


def tq_pack_lowrank_q(U, V, out=None):
    """Quantise (per column, 4 bits) and lay out the low-rank factors U (d x r), V (r x m) for tq_linear_qlr."""
    lib = load()
    _need_cuda(U, V)
    d, r = U.shape
    m = V.shape[1]
    if out is None:
        out = torch.empty(lib.tq_lowrank_q_bytes(d, m, r), dtype=torch.uint8, device=U.device)
    _check("tq_pack_lowrank_q", lib.tq_pack_lowrank_q(_p(U), _p(V), _dt(U), d, m, r, _p(out), _stream(U)))
    return out


def tq_linear_qlr_workspace_bytes(n: int, d: int, r: int) -> int:
    return load().tq_linear_qlr_workspace_bytes(n, d, r)


def tq_linear_qlr_workspace_offsets(n: int, d: int, r: int) -> dict:
    """Byte offsets of s_x, the activation codes, s_t and the first-stage codes inside tq_linear_qlr's workspace."""
    off = (ctypes.c_size_t * 4)()
    _check("tq_linear_qlr_workspace_offsets", load().tq_linear_qlr_workspace_offsets(n, d, r, off))
    return {"s_x": off[0], "x_codes": off[1], "s_t": off[2], "t_codes": off[3]}


def tq_linear_qlr(X, w_codes, s_w, lowrank_q, m: int, r: int, y_dtype=torch.bfloat16, Y=None, ws=None, acc=None,
                  acc2=None):
    """Y = s_x s_w (Q4(X) Q4(R)) + (s_x s_t) s_v (Q4(T) Q4(V)), T the per-token re-quantised Q4(X) Q4(U).
    acc / acc2 (n x m int32, optional): the kernel's exact residual and second-stage sums, through
    tq_linear_qlr_debug."""
    lib = load()
    _need_cuda(X, w_codes, s_w, lowrank_q, Y, ws, acc, acc2)
    n, d = X.shape
    if Y is None:
        Y = torch.empty((n, m), dtype=y_dtype, device=X.device)
    if ws is None:
        ws = torch.empty(max(1, tq_linear_qlr_workspace_bytes(n, d, r)), dtype=torch.uint8, device=X.device)
    if acc is not None:
        _check("tq_linear_qlr_debug", lib.tq_linear_qlr_debug(_p(X), _dt(X), n, d, m, r, _p(w_codes), _p(s_w),
                                                              _p(lowrank_q), _p(Y), _dt(Y), _p(ws), ws.numel(),
                                                              _p(acc), _p(acc2), _stream(X)))
    else:
        _check("tq_linear_qlr", lib.tq_linear_qlr(_p(X), _dt(X), n, d, m, r, _p(w_codes), _p(s_w), _p(lowrank_q),
                                                  _p(Y), _dt(Y), _p(ws), ws.numel(), _stream(X)))
    return Y


def tq_weight_colsum(w_codes, k: int, bits: int = 4, colsum=None):
    """Sum of each code row of a packed weight (m rows of k codes) -> int32 m."""
    lib = load()
    _need_cuda(w_codes, colsum)
    m = w_codes.shape[0]
    if colsum is None:
        colsum = torch.empty(m, dtype=torch.int32, device=w_codes.device)
    _check("tq_weight_colsum", lib.tq_weight_colsum(_p(w_codes), m, k, bits, _p(colsum), _stream(w_codes)))
    return colsum


def tq_linear_mp_asym_workspace_bytes(n: int, d: int, d_hi: int) -> int:
    return load().tq_linear_mp_asym_workspace_bytes(n, d, d_hi)


def tq_linear_mp_asym_workspace_offsets(n: int, d: int, d_hi: int) -> dict:
    off = (ctypes.c_size_t * 6)()
    _check("tq_linear_mp_asym_workspace_offsets", load().tq_linear_mp_asym_workspace_offsets(n, d, d_hi, off))
    return {"s_xl": off[0], "s_xh": off[1], "x_codes_l": off[2], "x_codes_h": off[3], "z_xl": off[4], "z_xh": off[5]}


def tq_linear_mp_asym(Xrot, d_hi: int, wl_codes, s_wl, colsum_l, wh_codes, s_wh, colsum_h, m: int,
                      y_dtype=torch.bfloat16, Y=None, ws=None, acc_l=None, acc_h=None):
    """tq_linear_mp with per-token asymmetric activations (zero-points), weights symmetric per channel.
    acc_l / acc_h (optional): the kernel's exact sums of the stored codes, through tq_linear_mp_asym_debug."""
    lib = load()
    _need_cuda(Xrot, wl_codes, s_wl, colsum_l, wh_codes, s_wh, colsum_h, Y, ws, acc_l, acc_h)
    n, d = Xrot.shape
    if Y is None:
        Y = torch.empty((n, m), dtype=y_dtype, device=Xrot.device)
    if ws is None:
        ws = torch.empty(max(1, tq_linear_mp_asym_workspace_bytes(n, d, d_hi)), dtype=torch.uint8,
                         device=Xrot.device)
    if acc_l is not None:
        _check("tq_linear_mp_asym_debug", lib.tq_linear_mp_asym_debug(
            _p(Xrot), _dt(Xrot), n, d, m, d_hi, _p(wl_codes), _p(s_wl), _p(colsum_l), _p(wh_codes), _p(s_wh),
            _p(colsum_h), _p(Y), _dt(Y), _p(ws), ws.numel(), _p(acc_l), _p(acc_h), _stream(Xrot)))
    else:
        _check("tq_linear_mp_asym", lib.tq_linear_mp_asym(_p(Xrot), _dt(Xrot), n, d, m, d_hi, _p(wl_codes),
                                                          _p(s_wl), _p(colsum_l), _p(wh_codes), _p(s_wh),
                                                          _p(colsum_h), _p(Y), _dt(Y), _p(ws), ws.numel(),
                                                          _stream(Xrot)))
    return Y


def tq_linear_asym_workspace_offsets(n: int, d: int, m: int, r: int) -> dict:
    off = (ctypes.c_size_t * 4)()
    _check("tq_linear_asym_workspace_offsets", load().tq_linear_asym_workspace_offsets(n, d, m, r, off))
    return {"s_x": off[0], "x_codes": off[1], "z_x": off[2], "T": off[3]}


def tq_linear_asym(X, w_codes, s_w, colsum, lowrank, m: int, r: int, y_dtype=torch.bfloat16, Y=None, ws=None,
                   acc=None):
    """tq_linear with per-token asymmetric activations; colsum = tq_weight_colsum(w_codes, d, 4).
    acc (optional): the kernel's exact sums of the stored codes (u - 8), through tq_linear_asym_debug."""
    lib = load()
    _need_cuda(X, w_codes, s_w, colsum, lowrank, Y, ws, acc)
    n, d = X.shape
    if Y is None:
        Y = torch.empty((n, m), dtype=y_dtype, device=X.device)
    if ws is None:
        ws = torch.zeros(max(1, lib.tq_linear_asym_workspace_bytes(n, d, m, r)), dtype=torch.uint8, device=X.device)
    if acc is not None:
        _check("tq_linear_asym_debug", lib.tq_linear_asym_debug(_p(X), _dt(X), n, d, m, r, _p(w_codes), _p(s_w),
                                                                _p(colsum), _p(lowrank), _p(Y), _dt(Y), _p(ws),
                                                                ws.numel(), _p(acc), _stream(X)))
    else:
        _check("tq_linear_asym", lib.tq_linear_asym(_p(X), _dt(X), n, d, m, r, _p(w_codes), _p(s_w), _p(colsum),
                                                    _p(lowrank), _p(Y), _dt(Y), _p(ws), ws.numel(), _stream(X)))
    return Y


def tq_debug_accumulate(x_codes, w_codes, k: int, bits: int = 4, acc=None):
    """Exact int32 product of code matrices (x n x k, w m x k) -> n x m."""
    lib = load()
    _need_cuda(x_codes, w_codes, acc)
    n, m = x_codes.shape[0], w_codes.shape[0]
    if acc is None:
        acc = torch.empty((n, m), dtype=torch.int32, device=x_codes.device)
    _check("tq_debug_accumulate", lib.tq_debug_accumulate(_p(x_codes), _p(w_codes), n, k, m, bits, _p(acc),
                                                          _stream(x_codes)))
    return acc


def tq_debug_accumulate_i8(x_codes, w_codes, k: int, acc=None):
    """Exact int32 product -> n x m from int8 activation codes in the tile GEMM's order (x n x k bytes) and
    nibble-packed weight codes (w m x k/2)."""
    lib = load()
    _need_cuda(x_codes, w_codes, acc)
    n, m = x_codes.shape[0], w_codes.shape[0]
    if acc is None:
        acc = torch.empty((n, m), dtype=torch.int32, device=x_codes.device)
    _check("tq_debug_accumulate_i8", lib.tq_debug_accumulate_i8(_p(x_codes), _p(w_codes), n, k, m, _p(acc),
                                                                _stream(x_codes)))
    return acc


def tq_debug_gemm_w4a4(x_codes, x_packed: bool, s_x, w_codes, s_w, k: int, Y=None):
    """bf16 Y = s_x s_w (C_x C_w^T) through the tile GEMM on nibble-packed (x_packed) or int8 (tile order)
    activation codes."""
    lib = load()
    _need_cuda(x_codes, s_x, w_codes, s_w, Y)
    n, m = x_codes.shape[0], w_codes.shape[0]
    if Y is None:
        Y = torch.empty((n, m), dtype=torch.bfloat16, device=x_codes.device)
    _check("tq_debug_gemm_w4a4", lib.tq_debug_gemm_w4a4(_p(x_codes), 1 if x_packed else 0, _p(s_x), _p(w_codes),
                                                        _p(s_w), n, k, m, _p(Y), _stream(x_codes)))
    return Y


def tq_profile_enable(on: bool = True):
    _check("tq_profile_enable", load().tq_profile_enable(1 if on else 0))


def tq_profile_reset():
    _check("tq_profile_reset", load().tq_profile_reset())


def tq_profile_read() -> dict:
    """{kernel name: (launches, total ms)} of the launches recorded while enabled."""
    lib = load()
    buf = (KernelStat * 64)()
    k = lib.tq_profile_read(buf, 64)
    if k < 0:
        raise TQError("tq_profile_read", k)
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(k, 64))}

"""C ABI checks that need no GPU: the library loads, exports every entry point
that include/tq.h declares, and rejects bad arguments before any HIP call."""

from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")

from rank_augmented_quantized_amd import tq as tqb  # noqa: E402


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tqb.LIB):
        pytest.skip("libtq.so not built (run __graft_entry__.build())")
    return tqb.load()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(tqb.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", tqb.LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\S+)$", out, flags=re.M))
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings_and_version(lib):
    assert lib.tq_version() == 106
    for code in range(-7, 1):
        assert lib.tq_status_string(code)
    assert b"unknown" in lib.tq_status_string(-99)


def test_size_queries(lib):
    assert lib.tq_codes_bytes(3, 64, 4) == 96
    assert lib.tq_codes_bytes(3, 64, 8) == 192
    assert lib.tq_codes_bytes(3, 63, 4) == 0
    assert lib.tq_codes_bytes(3, 64, 5) == 0
    # packed low-rank: r padded to a power of two >= 32
    assert lib.tq_lowrank_bytes(512, 512, 16) == (32 * 512 + 512 * 32) * 2
    assert lib.tq_lowrank_bytes(4096, 14336, 64) == (64 * 4096 + 14336 * 64) * 2
    assert lib.tq_lowrank_bytes(512, 512, 257) == 0
    ws = lib.tq_linear_workspace_bytes(16, 512, 512, 16)
    assert ws >= 256 + 16 * 4 + 16 * 256 + 16 * 32 * 2
    off = tqb.tq_linear_workspace_offsets(16, 512, 512, 16)
    assert off["s_x"] >= 256 and off["x_codes"] >= off["s_x"] + 64 and off["T"] >= off["x_codes"] + 16 * 256
    assert all(v % 256 == 0 for v in off.values())
    assert lib.tq_linear_mp_workspace_bytes(8, 256, 64) >= 8 * 96 + 8 * 64 + 64


# Fake, aligned, non-null device addresses: every call below must fail its
# argument check and return before touching them.
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10008)
NUL = None
S = None  # null stream


def test_pack_weight_validation(lib):
    assert lib.tq_pack_weight(A, 0, 512, 64, 5, B, C, S) == -4
    assert lib.tq_pack_weight(A, 7, 512, 64, 4, B, C, S) == -3
    assert lib.tq_pack_weight(A, 0, 100, 64, 4, B, C, S) == -2
    assert lib.tq_pack_weight(A, 0, 512, 0, 4, B, C, S) == -2
    assert lib.tq_pack_weight(NUL, 0, 512, 64, 4, B, C, S) == -1
    assert lib.tq_pack_weight(A, 0, 512, 64, 4, MIS, C, S) == -5


def test_quantize_act_validation(lib):
    assert lib.tq_quantize_act(A, 1, 0, 512, 4, NUL, NUL, S) == 0  # n == 0 is a no-op
    assert lib.tq_quantize_act(A, 1, 4, 48, 4, B, C, S) == -2  # d % 32
    assert lib.tq_quantize_act(A, 1, 4, 48, 8, MIS, C, S) == -5  # 8 bits accepts d % 16
    assert lib.tq_quantize_act(A, 1, -1, 512, 4, B, C, S) == -2
    assert lib.tq_quantize_act(A, 1, 4, 512, 3, B, C, S) == -4
    assert lib.tq_quantize_act(A, 1, 4, 512, 4, B, NUL, S) == -1


def test_linear_validation(lib):
    n, d, m, r = 64, 512, 256, 16
    need = lib.tq_linear_workspace_bytes(n, d, m, r)
    assert lib.tq_linear(A, 2, n, d, m, r, B, C, A, B, 1, C, need, S) == -3
    assert lib.tq_linear(A, 1, n, 500, m, r, B, C, A, B, 1, C, need, S) == -2
    assert lib.tq_linear(A, 1, n, d, m, 300, B, C, A, B, 1, C, need, S) == -2
    assert lib.tq_linear(A, 1, n, d, 0, r, B, C, A, B, 1, C, need, S) == -2
    assert lib.tq_linear(A, 1, n, d, m, r, B, C, NUL, B, 1, C, need, S) == -1  # r > 0 needs the low-rank factors
    assert lib.tq_linear(A, 1, n, d, m, r, B, C, A, NUL, 1, C, need, S) == -1
    assert lib.tq_linear(A, 1, n, d, m, r, B, C, A, B, 1, MIS, need, S) == -5
    assert lib.tq_linear(A, 1, n, d, m, r, B, C, A, B, 1, C, need - 1, S) == -6
    assert lib.tq_linear(A, 1, 0, d, m, r, NUL, NUL, NUL, NUL, 1, NUL, 0, S) == 0


def _ms(*v):
    return (ctypes.c_int64 * len(v))(*v)


def test_group_size_queries(lib):
    # gate/up: two layers of r 64 -> T of 128 columns, L2^T of all channels at r_pad 64
    assert lib.tq_lowrank_group_bytes(4096, _ms(14336, 14336), 2, 64) == (128 * 4096 + 28672 * 64) * 2
    # three layers of r 32: 96 T columns rounded up to 128
    assert lib.tq_lowrank_group_bytes(512, _ms(512, 256, 256), 3, 32) == (128 * 512 + 1024 * 32) * 2
    assert lib.tq_lowrank_group_bytes(512, _ms(300, 256), 2, 32) == 0  # a layer before the last off the 256 grid
    assert lib.tq_lowrank_group_bytes(512, _ms(256, 300), 2, 32) == (64 * 512 + 556 * 32) * 2
    assert lib.tq_lowrank_group_bytes(512, _ms(256, 256, 256), 3, 128) == 0  # 3 x 128 T columns > 256
    assert lib.tq_lowrank_group_bytes(512, _ms(*([256] * 9)), 9, 16) == 0  # more than 8 layers
    # the workspace of a group is that of one layer as wide as all of them with the group's T width
    assert lib.tq_linear_group_workspace_bytes(64, 512, _ms(256, 256), 2, 64) == \
        lib.tq_linear_workspace_bytes(64, 512, 512, 128)
    assert lib.tq_linear_group_workspace_bytes(64, 512, _ms(256), 1, 16) == lib.tq_linear_workspace_bytes(64, 512, 256, 16)


def test_linear_group_validation(lib):
    n, d, r = 64, 512, 16
    ms = _ms(256, 512)
    need = lib.tq_linear_group_workspace_bytes(n, d, ms, 2, r)
    assert lib.tq_linear_group(A, 1, n, d, ms, 2, r, B, C, A, B, 1, C, need - 1, S) == -6
    assert lib.tq_linear_group(A, 1, n, d, _ms(200, 256), 2, r, B, C, A, B, 1, C, need, S) == -2
    assert lib.tq_linear_group(A, 1, n, d, ms, 0, r, B, C, A, B, 1, C, need, S) == -2
    assert lib.tq_linear_group(A, 1, n, d, NUL, 2, r, B, C, A, B, 1, C, need, S) == -1
    assert lib.tq_linear_group(A, 1, n, d, ms, 2, r, B, C, NUL, B, 1, C, need, S) == -1
    assert lib.tq_linear_group(A, 1, n, d, ms, 2, r, B, C, A, B, 1, MIS, need, S) == -5
    assert lib.tq_linear_group(A, 2, n, d, ms, 2, r, B, C, A, B, 1, C, need, S) == -3
    assert lib.tq_linear_group(A, 1, 0, d, ms, 2, r, NUL, NUL, NUL, NUL, 1, NUL, 0, S) == 0
    L = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    Ln = (ctypes.c_void_p * 2)(0x10000, None)
    assert lib.tq_pack_lowrank_group(L, L, 1, d, ms, 2, r, MIS, S) == -5
    assert lib.tq_pack_lowrank_group(L, Ln, 1, d, ms, 2, r, A, S) == -1
    assert lib.tq_pack_lowrank_group(L, L, 1, d, ms, 2, 0, A, S) == -2
    assert lib.tq_pack_lowrank_group(L, L, 5, d, ms, 2, r, A, S) == -3


def test_rht_validation(lib):
    assert lib.tq_rht_bytes(8192) == 1024 + 2 * 8192  # sign bits, then uint16 positions
    assert lib.tq_rht_bytes(130) == 0 and lib.tq_rht_bytes(16384) == 0
    assert lib.tq_pack_rht(A, B, 200, C, S) == -2
    assert lib.tq_pack_rht(NUL, B, 256, C, S) == -1
    assert lib.tq_pack_rht(A, B, 256, MIS, S) == -5
    n, d, dh, m = 8, 512, 128, 64
    need = lib.tq_linear_mp_workspace_bytes(n, d, dh)
    assert lib.tq_linear_mp_rht(A, 1, n, 544, m, 160, B, A, B, C, A, B, 1, C, need, S) == -2  # d % 128
    assert lib.tq_linear_mp_rht(A, 1, n, 16384, m, 128, B, A, B, C, A, B, 1, C, need, S) == -2
    assert lib.tq_linear_mp_rht(A, 1, n, d, m, dh, NUL, A, B, C, A, B, 1, C, need, S) == -1
    assert lib.tq_linear_mp_rht(A, 1, n, d, m, dh, MIS, A, B, C, A, B, 1, C, need, S) == -5
    assert lib.tq_linear_mp_rht(A, 1, n, d, m, dh, B, A, B, C, A, B, 1, C, need - 1, S) == -6
    assert lib.tq_linear_mp_rht(A, 1, 0, d, m, dh, NUL, A, B, C, A, B, 1, C, 0, S) == 0
    off = tqb.tq_linear_mp_workspace_offsets(n, d, dh)
    assert off["x_codes_h"] >= off["x_codes_l"] + n * (d - dh) and all(v % 256 == 0 for v in off.values())


def test_qlr_validation(lib):
    # packed factors: U^T codes r_pad x d/2, s_u r_pad, V^T codes m x r_pad/2, s_v m (256-byte aligned parts)
    assert lib.tq_lowrank_q_bytes(512, 256, 32) == 32 * 256 + 256 + 256 * 16 + 1024
    assert lib.tq_lowrank_q_bytes(512, 256, 0) == 0 and lib.tq_lowrank_q_bytes(512, 256, 257) == 0
    assert lib.tq_pack_lowrank_q(A, B, 1, 520, 256, 32, C, S) == -2  # d % 32
    assert lib.tq_pack_lowrank_q(A, B, 1, 512, 256, 0, C, S) == -2
    assert lib.tq_pack_lowrank_q(A, NUL, 1, 512, 256, 32, C, S) == -1
    assert lib.tq_pack_lowrank_q(A, B, 1, 512, 256, 32, MIS, S) == -5
    assert lib.tq_pack_lowrank_q(A, B, 7, 512, 256, 32, C, S) == -3
    n, d, m, r = 64, 512, 256, 32
    need = lib.tq_linear_qlr_workspace_bytes(n, d, r)
    assert need == 256 + n * d + 256 + n * 32
    assert lib.tq_linear_qlr(A, 1, n, d, m, 0, B, C, A, B, 1, C, need, S) == -2  # r < 1
    assert lib.tq_linear_qlr(A, 1, n, 520, m, r, B, C, A, B, 1, C, need, S) == -2
    assert lib.tq_linear_qlr(A, 1, n, d, m, r, B, C, NUL, B, 1, C, need, S) == -1
    assert lib.tq_linear_qlr(A, 1, n, d, m, r, B, C, A, MIS, 1, C, need, S) == -5
    assert lib.tq_linear_qlr(A, 1, n, d, m, r, B, C, A, B, 1, C, need - 1, S) == -6
    assert lib.tq_linear_qlr(A, 1, 0, d, m, r, B, C, A, B, 1, C, 0, S) == 0
    off = tqb.tq_linear_qlr_workspace_offsets(n, d, r)
    assert off["x_codes"] >= off["s_x"] + 4 * n and off["t_codes"] >= off["s_t"] + 4 * n
    assert all(v % 256 == 0 for v in off.values())


def test_linear_asym_validation(lib):
    n, d, m, r = 64, 512, 256, 32
    need = lib.tq_linear_asym_workspace_bytes(n, d, m, r)
    assert need > lib.tq_linear_workspace_bytes(n, d, m, r)
    assert lib.tq_linear_asym(A, 1, n, 520, m, r, B, C, A, B, A, 1, C, need, S) == -2
    assert lib.tq_linear_asym(A, 1, n, 32768, m, r, B, C, A, B, A, 1, C, need, S) == -2  # d > 16384
    assert lib.tq_linear_asym(A, 1, n, d, m, r, B, C, NUL, B, A, 1, C, need, S) == -1  # colsum
    assert lib.tq_linear_asym(A, 1, n, d, m, r, B, C, MIS, B, A, 1, C, need, S) == -5
    assert lib.tq_linear_asym(A, 1, n, d, m, r, B, C, A, B, A, 1, C, need - 1, S) == -6
    assert lib.tq_linear_asym(A, 1, 0, d, m, r, B, C, A, B, A, 1, C, 0, S) == 0
    off = tqb.tq_linear_asym_workspace_offsets(n, d, m, r)
    assert off["x_codes"] >= off["s_x"] + 4 * n and off["z_x"] >= off["T"] and all(v % 256 == 0 for v in off.values())


def test_mp_bits_validation(lib):
    assert lib.tq_codes_bytes(4, 64, 3) == 4 * 32 and lib.tq_codes_bytes(4, 64, 6) == 4 * 64
    assert lib.tq_codes_bytes(4, 64, 5) == 0
    assert lib.tq_pack_weight(A, 1, 512, 64, 5, B, C, S) == -4
    assert lib.tq_pack_weight(A, 1, 48, 64, 3, B, C, S) == -2  # 3-bit rows: d % 32
    n, d, dh, m = 64, 512, 64, 256
    need = lib.tq_linear_mp_workspace_bytes(n, d, dh)
    assert lib.tq_linear_mp_bits(A, 1, n, d, m, dh, 4, 6, B, C, A, B, C, 1, A, need, S) == -4
    assert lib.tq_linear_mp_bits(A, 1, n, d, m, dh, 3, 8, B, C, A, B, C, 1, A, need, S) == -4
    assert lib.tq_linear_mp_bits(A, 1, n, d, m, 40, 3, 6, B, C, A, B, C, 1, A, need, S) == -2
    assert lib.tq_linear_mp_bits(A, 1, n, d, m, dh, 3, 6, B, C, A, B, C, 1, A, need - 1, S) == -6
    assert lib.tq_linear_mp_bits(A, 1, 0, d, m, dh, 3, 6, B, C, A, B, C, 1, A, 0, S) == 0


def test_mp_asym_validation(lib):
    assert lib.tq_weight_colsum(A, 8, 48, 4, C, S) == -2  # k % 32
    assert lib.tq_weight_colsum(A, 8, 64, 6, C, S) == -4
    assert lib.tq_weight_colsum(NUL, 8, 64, 4, C, S) == -1
    assert lib.tq_weight_colsum(A, 8, 64, 4, MIS, S) == -5
    n, d, dh, m = 64, 512, 64, 256
    need = lib.tq_linear_mp_asym_workspace_bytes(n, d, dh)
    assert need == lib.tq_linear_mp_workspace_bytes(n, d, dh) + 2 * 256
    assert lib.tq_linear_mp_asym(A, 1, n, d, m, 40, B, C, A, A, B, C, A, 1, C, need, S) == -2  # d_hi % 16
    assert lib.tq_linear_mp_asym(A, 1, n, 32768, m, 128, B, C, A, A, B, C, A, 1, C, need, S) == -2  # d > 16384
    assert lib.tq_linear_mp_asym(A, 1, n, d, m, dh, B, C, NUL, A, B, C, A, 1, C, need, S) == -1  # colsum_l
    assert lib.tq_linear_mp_asym(A, 1, n, d, m, dh, B, C, A, A, B, NUL, A, 1, C, need, S) == -1  # colsum_h
    assert lib.tq_linear_mp_asym(A, 1, n, d, m, dh, B, C, MIS, A, B, C, A, 1, C, need, S) == -5
    assert lib.tq_linear_mp_asym(A, 1, n, d, m, dh, B, C, A, A, B, C, A, 1, C, need - 1, S) == -6
    assert lib.tq_linear_mp_asym(A, 1, 0, d, m, dh, B, C, A, A, B, C, A, 1, C, 0, S) == 0
    off = tqb.tq_linear_mp_asym_workspace_offsets(n, d, dh)
    assert off["z_xl"] >= off["x_codes_h"] + n * dh and off["z_xh"] >= off["z_xl"] + 4 * n
    assert all(v % 256 == 0 for v in off.values())


def test_linear_mp_validation(lib):
    n, d, dh, m = 64, 512, 64, 256
    need = lib.tq_linear_mp_workspace_bytes(n, d, dh)
    assert lib.tq_linear_mp(A, 1, n, d, m, 40, B, C, A, B, C, 1, A, need, S) == -2  # d_hi % 16
    assert lib.tq_linear_mp(A, 1, n, 520, m, 64, B, C, A, B, C, 1, A, need, S) == -2  # (d - d_hi) % 32
    assert lib.tq_linear_mp(A, 1, n, d, m, d + 16, B, C, A, B, C, 1, A, need, S) == -2
    assert lib.tq_linear_mp(A, 1, n, d, m, dh, B, C, NUL, B, C, 1, A, need, S) == -1
    assert lib.tq_linear_mp(A, 1, n, d, m, dh, B, C, A, B, C, 1, A, need - 1, S) == -6


def test_debug_entry_points_validation(lib):
    """The accumulator-export variants check their export buffers after the layer's own checks."""
    n, d, m, r = 64, 512, 256, 16
    need = lib.tq_linear_workspace_bytes(n, d, m, r)
    assert lib.tq_linear_debug(A, 1, n, d, m, r, B, C, A, B, 1, C, need, NUL, S) == -1
    assert lib.tq_linear_debug(A, 1, n, d, m, r, B, C, A, B, 1, C, need, MIS, S) == -5
    assert lib.tq_linear_debug(A, 1, n, 500, m, r, B, C, A, B, 1, C, need, A, S) == -2
    assert lib.tq_linear_debug(A, 1, 0, d, m, r, NUL, NUL, NUL, NUL, 1, NUL, 0, NUL, S) == 0
    dh = 64
    need = lib.tq_linear_mp_workspace_bytes(n, d, dh)
    assert lib.tq_linear_mp_bits_debug(A, 1, n, d, m, dh, 4, 8, B, C, A, B, C, 1, A, need, A, NUL, S) == -1
    assert lib.tq_linear_mp_bits_debug(A, 1, n, d, m, 0, 4, 8, B, C, NUL, NUL, C, 1, A, need, NUL, NUL, S) == -1
    assert lib.tq_linear_mp_bits_debug(A, 1, n, d, m, dh, 4, 8, B, C, A, B, C, 1, A, need, A, MIS, S) == -5
    assert lib.tq_linear_mp_bits_debug(A, 1, n, d, m, dh, 4, 6, B, C, A, B, C, 1, A, need, A, B, S) == -4
    need = lib.tq_linear_mp_asym_workspace_bytes(n, d, dh)
    assert lib.tq_linear_mp_asym_debug(A, 1, n, d, m, dh, B, C, A, A, B, C, A, 1, C, need, NUL, B, S) == -1
    need = lib.tq_linear_asym_workspace_bytes(n, d, m, r)
    assert lib.tq_linear_asym_debug(A, 1, n, d, m, r, B, C, A, B, A, 1, C, need, MIS, S) == -5
    need = lib.tq_linear_qlr_workspace_bytes(n, d, r)
    assert lib.tq_linear_qlr_debug(A, 1, n, d, m, r, B, C, A, B, 1, C, need, A, NUL, S) == -1
    assert lib.tq_linear_qlr_debug(A, 1, n, d, m, 0, B, C, A, B, 1, C, need, A, B, S) == -2


def test_debug_accumulate_validation(lib):
    assert lib.tq_debug_accumulate(A, B, 4, 48, 8, 4, C, S) == -2
    assert lib.tq_debug_accumulate(A, B, 4, 64, 8, 6, C, S) == -4
    assert lib.tq_debug_accumulate(A, NUL, 4, 64, 8, 4, C, S) == -1
    assert lib.tq_debug_accumulate(A, B, 4, 64, 8, 4, MIS, S) == -5


def test_profile_record_without_launches(lib):
    assert lib.tq_profile_reset() == 0
    assert lib.tq_profile_enable(1) == 0
    assert tqb.tq_profile_read() == {}
    assert lib.tq_profile_enable(0) == 0


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(tqb, "_lib", None)
    with pytest.raises(ImportError, match="missing"):
        tqb.load(str(tmp_path / "nope.so"))


@pytest.mark.parametrize("n,d,m,r", [(1, 512, 256, 32), (17, 4096, 1024, 64), (33, 14336, 4096, 100),
                                     (1030, 2048, 512, 0), (4096, 4096, 4096, 256)])
def test_workspace_regions_fit_and_do_not_overlap(lib, n, d, m, r):
    """Every region the offset queries report lies inside the reported workspace size, 256-byte aligned, and the
    regions do not overlap (sizes from the layouts documented in include/tq.h)."""
    rp = 0 if r == 0 else max(32, 1 << (r - 1).bit_length())
    small = n <= 32

    def check(total, regions):
        regions = sorted(regions)
        for (o, sz), (o2, _) in zip(regions, regions[1:]):
            assert o % 256 == 0 and o + sz <= o2, (regions,)
        assert regions[-1][0] + regions[-1][1] <= total

    off = tqb.tq_linear_workspace_offsets(n, d, m, r)
    check(lib.tq_linear_workspace_bytes(n, d, m, r),
          [(off["s_x"], 4 * n), (off["x_codes"], n * (d // 2 if small else d)), (off["T"], n * rp * 2)])
    if r:
        off = tqb.tq_linear_qlr_workspace_offsets(n, d, r)
        check(lib.tq_linear_qlr_workspace_bytes(n, d, r),
              [(off["s_x"], 4 * n), (off["x_codes"], n * d), (off["s_t"], 4 * n), (off["t_codes"], n * rp)])
    off = tqb.tq_linear_asym_workspace_offsets(n, d, m, r)
    check(lib.tq_linear_asym_workspace_bytes(n, d, m, r),
          [(off["s_x"], 4 * n), (off["x_codes"], n * (d // 2 if small else d)), (off["z_x"], 4 * n),
           (off["T"], n * rp * 2)])
    dh = 128 if d >= 256 else 0
    off = tqb.tq_linear_mp_asym_workspace_offsets(n, d, dh)
    check(lib.tq_linear_mp_asym_workspace_bytes(n, d, dh),
          [(off["s_xl"], 4 * n), (off["s_xh"], 4 * n), (off["x_codes_l"], n * (d - dh)), (off["x_codes_h"], n * dh),
           (off["z_xl"], 4 * n), (off["z_xh"], 4 * n)])


def test_counter_block_is_at_fixed_offsets(lib):
    """The hand-off words and counters that must be zero before a call sit in the first 8 KiB of the workspace
    whatever the shape, and no other region of tq_linear or tq_linear_asym reaches into them: one workspace,
    zero-filled once, can serve calls of any shape in turn (and the no-alloc scratch clears 64 KiB once)."""
    shapes = [(1, 512, 256, 32), (5, 2048, 200, 64), (16, 4096, 14336, 64), (8, 14336, 4096, 64), (33, 256, 130, 0),
              (200, 1024, 384, 64), (256, 4096, 14336, 64), (1030, 544, 96, 128), (4096, 4096, 4096, 32)]
    for n, d, m, r in shapes:
        off = tqb.tq_linear_workspace_offsets(n, d, m, r)
        assert off["sync"] == 0
        assert min(off["s_x"], off["x_codes"], off["T"]) >= 8192, (n, d, m, r, off)
        aoff = tqb.tq_linear_asym_workspace_offsets(n, d, m, r)
        assert min(aoff.values()) >= 8192, (n, d, m, r, aoff)


def test_boundary_departures_are_enforced(lib):
    """Each documented difference from the survey's boundary, checked where it is decided (before any HIP call)."""
    n, m, r = 8, 256, 16
    # d: a multiple of 32 (the MFMA k-step), not merely even
    for d in (34, 48, 100, 4080):
        need = lib.tq_linear_workspace_bytes(n, 4096, m, r)
        assert lib.tq_linear(A, 1, n, d, m, r, B, C, A, B, 1, C, need, S) == -2, d
    assert lib.tq_linear_workspace_bytes(n, 34, m, r) == 0
    d = 512
    need = lib.tq_linear_workspace_bytes(n, d, m, r)
    # the low-rank factors come as one packed buffer (tq_pack_lowrank), NULL iff r == 0
    assert lib.tq_linear(A, 1, n, d, m, r, B, C, NUL, B, 1, C, need, S) == -1
    assert lib.tq_linear(A, 1, n, d, m, r, B, C, MIS, B, 1, C, need, S) == -5
    # the workspace is caller-owned and sized by the query; one byte short is refused
    assert lib.tq_linear(A, 1, n, d, m, r, B, C, A, B, 1, C, need - 1, S) == -6
    # tq_linear_mp takes (n, d, m, d_hi) in the survey's order: d_hi past d, or not a multiple of 16, is a shape error
    dh = 64
    need_mp = lib.tq_linear_mp_workspace_bytes(n, d, dh)
    assert lib.tq_linear_mp(A, 1, n, d, m, d + 16, B, C, A, B, B, 1, C, need_mp, S) == -2
    assert lib.tq_linear_mp(A, 1, n, d, m, 40, B, C, A, B, B, 1, C, need_mp, S) == -2
    assert lib.tq_linear_mp(A, 1, n, d, 0, dh, B, C, A, B, B, 1, C, need_mp, S) == -2
    assert lib.tq_linear_mp(A, 1, 0, d, m, dh, NUL, NUL, NUL, NUL, NUL, 1, NUL, 0, S) == 0


def test_stream_read_validation(lib):
    out = ctypes.c_void_p(0x40000)
    assert lib.tq_debug_stream_read(NUL, 1024, out, 4, S) == -1
    assert lib.tq_debug_stream_read(A, 1024, NUL, 4, S) == -1
    assert lib.tq_debug_stream_read(MIS, 1024, out, 4, S) == -5
    assert lib.tq_debug_stream_read(A, 1000, out, 4, S) == -5  # bytes not a multiple of 16
    assert lib.tq_debug_stream_read(A, 1024, out, 0, S) == -2
    assert lib.tq_debug_stream_read(A, 1024, out, 70000, S) == -2


def test_accumulate_i8_validation(lib):
    assert lib.tq_debug_accumulate_i8(NUL, B, 40, 64, 16, C, S) == -1
    assert lib.tq_debug_accumulate_i8(A, B, 40, 48, 16, C, S) == -2  # k not a multiple of 32
    assert lib.tq_debug_accumulate_i8(A, B, 40, 64, 0, C, S) == -2
    assert lib.tq_debug_accumulate_i8(MIS, B, 40, 64, 16, C, S) == -5
    assert lib.tq_debug_accumulate_i8(A, B, 0, 64, 16, NUL, S) == 0  # nothing to do


def test_gemm_w4a4_debug_validation(lib):
    assert lib.tq_debug_gemm_w4a4(A, 1, C, B, C, 40, 64, 16, NUL, S) == -1
    assert lib.tq_debug_gemm_w4a4(A, 0, NUL, B, C, 40, 64, 16, C, S) == -1
    assert lib.tq_debug_gemm_w4a4(A, 1, C, B, C, 40, 48, 16, C, S) == -2  # k not a multiple of 32
    assert lib.tq_debug_gemm_w4a4(MIS, 1, C, B, C, 40, 64, 16, C, S) == -5
    assert lib.tq_debug_gemm_w4a4(NUL, 1, NUL, NUL, NUL, 0, 64, 16, NUL, S) == 0  # nothing to do


def test_mfma_ceiling_validation(lib):
    out = ctypes.c_void_p(0x40000)
    assert lib.tq_debug_mfma_ceiling(16, 4, NUL, S) == -1
    assert lib.tq_debug_mfma_ceiling(0, 4, out, S) == -2
    assert lib.tq_debug_mfma_ceiling((1 << 20) + 1, 4, out, S) == -2
    assert lib.tq_debug_mfma_ceiling(16, 0, out, S) == -2
    assert lib.tq_debug_mfma_ceiling(16, 70000, out, S) == -2


def test_profiler_is_the_only_switchable_state(lib):
    """Timing is off unless enabled; with nothing recorded the read returns no entries, and reset clears it."""
    stats = (tqb.KernelStat * 8)()
    assert lib.tq_profile_reset() == 0
    assert lib.tq_profile_read(stats, 8) == 0
    assert lib.tq_profile_enable(1) == 0
    assert lib.tq_profile_read(stats, 8) == 0
    assert lib.tq_profile_enable(0) == 0
    assert lib.tq_profile_reset() == 0

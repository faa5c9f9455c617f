#!/usr/bin/env python3
"""Throughput of the rank-augmented W4A4 linear layer on one MI355X.

One step = one tq_linear call (per-token activation quantisation, first
low-rank stage, integer GEMM and the shared epilogue) on the Llama-3-8B
attention-projection workload (n = d = m = 4096, r = 32), inputs resident in
HBM.  Prints ONE JSON line (stdout); progress goes to stderr.

  value     effective int ops/s of the whole call, 2 n d m / t, in TOPS
  roofline  the integer GEMM kernel: algorithmic 2 n d m per launch over its
            average launch duration (HIP events on the launch stream, taken
            by the dispatch itself via hipExtLaunchKernelGGL), against the
            MI355X dense int8 MFMA peak (5.0 POP/s)
  cpu_baseline  the CPU oracle on the same workload (a bounded sample)
  sweep     the other workloads (decode rows against the 8 TB/s HBM peak,
            also with the calls captured in a HIP graph and replayed), and
            gate and up as one grouped call next to two separate calls
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tq_linear effective TOPS + % int8-MFMA peak (prefill); GB/s + % HBM (decode)"
PEAK_INT8_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_w4a4_attn_proj.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_augmented_quantized_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_hash: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_hash or "hbm_bytes_per_launch" not in kv:
        return None
    return float(kv["hbm_bytes_per_launch"])


def alg_bytes(n, d, m, r, x_bytes=2, y_bytes=2):
    """Bytes the layer itself must move: X, weight codes + scales, L1, L2, Y."""
    return n * d * x_bytes + d * m // 2 + 4 * m + 2 * d * r + 2 * r * m + y_bytes * n * m


def time_calls(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        fn(i)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def kernel_ms(fn, steps, torch, tq):
    """Per call, the time of each kernel name (dispatch timestamps; a name launched several times per call spans
    its first start to its last end)."""
    tq.tq_profile_reset()
    tq.tq_profile_enable(True)
    for i in range(steps):
        fn(i)
    torch.cuda.synchronize()
    stats = tq.tq_profile_read()
    tq.tq_profile_enable(False)
    tq.tq_profile_reset()
    return {k: v[1] / steps for k, v in stats.items()}


class LinearCase:
    """Device-resident inputs of one rank-augmented workload, with `copies`
    independent weight sets cycled through so that repeated calls stream the
    weights from HBM rather than from the last-level cache."""

    def __init__(self, wl, n, copies, torch, tq, dev):
        from workloads import draw_linear

        c = draw_linear(wl, n=n)
        self.n, self.d, self.m, self.r = n, wl.d, wl.m, wl.r
        xdt = torch.bfloat16 if wl.x_dtype == "bf16" else torch.float32
        self.x_bytes = 2 if wl.x_dtype == "bf16" else 4
        self.X = torch.from_numpy(c["X"]).to(dev).to(xdt)
        R = torch.from_numpy(c["R"]).to(dev)
        L1 = torch.from_numpy(c["L1"]).to(dev).bfloat16()
        L2 = torch.from_numpy(c["L2"]).to(dev).bfloat16()
        self.w = []
        for _ in range(copies):
            wc, sw = tq.tq_pack_weight(R, 4)
            lr = tq.tq_pack_lowrank(L1, L2) if self.r else None
            self.w.append((wc, sw, lr))
        del R
        self.Y = torch.empty((n, self.m), dtype=torch.bfloat16, device=dev)
        self.ws = tq.linear_workspace(n, self.d, self.m, self.r, dev)
        self.tq = tq

    def __call__(self, i):
        wc, sw, lr = self.w[i % len(self.w)]
        self.tq.tq_linear(self.X, wc, sw, lr, self.m, self.r, Y=self.Y, ws=self.ws)

    def graph_ms(self, torch, replays=20):
        """Per-call time with the calls (one per weight copy) captured in a HIP graph and replayed: the GPU time a
        serving loop that captures its decode step sees, without per-launch host overhead."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(len(self.w)):
                self(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(len(self.w)):
                self(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) / (replays * len(self.w))


class GroupCase:
    """Layers of one workload's shape that share X (gate and up), as one tq_linear_group call and, for
    comparison, as one tq_linear call per layer on the same device data; `copies` weight sets cycled."""

    def __init__(self, wl, n, groups, copies, torch, tq, dev):
        from workloads import draw_group

        c = draw_group(wl, n=n, groups=groups)
        self.n, self.d, self.m, self.r, self.G = n, wl.d, wl.m, wl.r, groups
        self.ms = [wl.m] * groups
        self.X = torch.from_numpy(c["X"]).to(dev).bfloat16()
        Rs = [torch.from_numpy(a).to(dev) for a in c["Rs"]]
        L1s = [torch.from_numpy(a).to(dev).bfloat16() for a in c["L1s"]]
        L2s = [torch.from_numpy(a).to(dev).bfloat16() for a in c["L2s"]]
        self.w = []
        for _ in range(copies):
            packed = [tq.tq_pack_weight(R, 4) for R in Rs]
            wc = torch.cat([p[0] for p in packed], dim=0).contiguous()
            sw = torch.cat([p[1] for p in packed]).contiguous()
            del packed
            lr = tq.tq_pack_lowrank_group(L1s, L2s)
            lrs = [tq.tq_pack_lowrank(L1s[g], L2s[g]) for g in range(groups)]
            self.w.append((wc, sw, lr, lrs))
        del Rs
        self.Y = torch.empty((n, groups * wl.m), dtype=torch.bfloat16, device=dev)
        self.Ys = [torch.empty((n, wl.m), dtype=torch.bfloat16, device=dev) for _ in range(groups)]
        self.ws = tq.linear_group_workspace(n, wl.d, self.ms, wl.r, dev)
        self.ws1 = tq.linear_workspace(n, wl.d, wl.m, wl.r, dev)
        self.tq = tq

    def __call__(self, i):
        wc, sw, lr, _ = self.w[i % len(self.w)]
        self.tq.tq_linear_group(self.X, wc, sw, lr, self.ms, self.r, Y=self.Y, ws=self.ws)

    def separate(self, i):
        wc, sw, _, lrs = self.w[i % len(self.w)]
        m = self.m
        for g in range(self.G):
            self.tq.tq_linear(self.X, wc[g * m:(g + 1) * m], sw[g * m:(g + 1) * m], lrs[g], m, self.r,
                              Y=self.Ys[g], ws=self.ws1)


class QlrCase:
    """The layer with its low-rank branch quantised too (tq_linear_qlr): Q(U), Q(V) packed from the workload's
    L1, L2; `copies` weight sets cycled."""

    def __init__(self, wl, n, copies, torch, tq, dev):
        from workloads import draw_linear

        c = draw_linear(wl, n=n)
        self.n, self.d, self.m, self.r = n, wl.d, wl.m, wl.r
        self.X = torch.from_numpy(c["X"]).to(dev).bfloat16()
        R = torch.from_numpy(c["R"]).to(dev)
        U = torch.from_numpy(c["L1"]).to(dev)
        V = torch.from_numpy(c["L2"]).to(dev)
        self.w = []
        for _ in range(copies):
            wc, sw = tq.tq_pack_weight(R, 4)
            self.w.append((wc, sw, tq.tq_pack_lowrank_q(U, V)))
        del R, U, V
        self.Y = torch.empty((n, self.m), dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(tq.tq_linear_qlr_workspace_bytes(n, self.d, self.r), dtype=torch.uint8, device=dev)
        self.tq = tq

    def __call__(self, i):
        wc, sw, lq = self.w[i % len(self.w)]
        self.tq.tq_linear_qlr(self.X, wc, sw, lq, self.m, self.r, Y=self.Y, ws=self.ws)


class AsymCase:
    """The rank-augmented layer with per-token asymmetric activations (tq_linear_asym); `copies` weight sets."""

    def __init__(self, wl, n, copies, torch, tq, dev):
        from workloads import draw_linear

        c = draw_linear(wl, n=n)
        self.n, self.d, self.m, self.r = n, wl.d, wl.m, wl.r
        self.X = torch.from_numpy(c["X"]).to(dev).bfloat16()
        R = torch.from_numpy(c["R"]).to(dev)
        L1 = torch.from_numpy(c["L1"]).to(dev).bfloat16()
        L2 = torch.from_numpy(c["L2"]).to(dev).bfloat16()
        self.w = []
        for _ in range(copies):
            wc, sw = tq.tq_pack_weight(R, 4)
            self.w.append((wc, sw, tq.tq_weight_colsum(wc, wl.d, 4), tq.tq_pack_lowrank(L1, L2)))
        del R
        self.Y = torch.empty((n, self.m), dtype=torch.bfloat16, device=dev)
        self.ws = torch.zeros(tq.load().tq_linear_asym_workspace_bytes(n, self.d, self.m, self.r), dtype=torch.uint8,
                              device=dev)
        self.tq = tq

    def __call__(self, i):
        wc, sw, cs, lr = self.w[i % len(self.w)]
        self.tq.tq_linear_asym(self.X, wc, sw, cs, lr, self.m, self.r, Y=self.Y, ws=self.ws)


class MpCase:
    """The two-subspace layer on pre-rotated X' (tq_linear_mp) or, with rht, on unrotated X with the rotation
    applied online inside the quantiser (tq_linear_mp_rht)."""

    def __init__(self, wl, torch, tq, dev, rht=False, asym=False, case=None, bits=(4, 8)):
        from workloads import draw_two_subspace

        c = case if case is not None else draw_two_subspace(wl)
        self.n, self.d, self.m, self.dh = wl.n, wl.d, wl.m, wl.d_hi
        dl = self.d - self.dh
        self.rht, self.asym, self.bits = rht, asym, tuple(bits)
        self.X = torch.from_numpy(c["X" if rht else "Xrot"]).to(dev).bfloat16()
        if rht:
            self.rot = tq.tq_pack_rht(torch.from_numpy(c["signs"].astype("float32")).to(dev),
                                      torch.from_numpy(c["perm"].astype("int32")).to(dev))
        W = torch.from_numpy(c["Wrot"])
        self.wl = tq.tq_pack_weight(W[:dl].contiguous().to(dev), self.bits[0])
        self.wh = tq.tq_pack_weight(W[dl:].contiguous().to(dev), self.bits[1])
        del W, c
        if asym:
            self.csl = tq.tq_weight_colsum(self.wl[0], dl, 4)
            self.csh = tq.tq_weight_colsum(self.wh[0], self.dh, 8)
        self.Y = torch.empty((self.n, self.m), dtype=torch.bfloat16, device=dev)
        wsb = (tq.tq_linear_mp_asym_workspace_bytes if asym else tq.tq_linear_mp_workspace_bytes)(self.n, self.d, self.dh)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        self.tq = tq

    def __call__(self, i):
        if self.asym:
            self.tq.tq_linear_mp_asym(self.X, self.dh, self.wl[0], self.wl[1], self.csl, self.wh[0], self.wh[1],
                                      self.csh, self.m, Y=self.Y, ws=self.ws)
        elif self.rht:
            self.tq.tq_linear_mp_rht(self.X, self.dh, self.rot, self.wl[0], self.wl[1], self.wh[0], self.wh[1], self.m,
                                     Y=self.Y, ws=self.ws)
        else:
            self.tq.tq_linear_mp(self.X, self.dh, self.wl[0], self.wl[1], self.wh[0], self.wh[1], self.m, Y=self.Y,
                                 ws=self.ws, bits=self.bits)


def stream_ceiling(torch, tq, dev, copies):
    """Read bandwidth of tq_debug_stream_read (the decode kernel's loads, nothing else): the weight codes of the
    Llama-3-8B MLP layers (29.4 MB, `copies` buffers cycled so that the last-level cache cannot serve them) and
    1 GiB, in GB/s."""
    out = []
    for nbytes, ncopy, blocks in ((4096 * 14336 // 2, copies, 1024), (1 << 30, 1, 4096)):
        bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(i + 1) for i in range(ncopy)]
        words = torch.empty(blocks, dtype=torch.int32, device=dev)
        for i in range(5):
            tq.tq_debug_stream_read(bufs[i % ncopy], words, blocks)
        torch.cuda.synchronize()
        steps = 64
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            tq.tq_debug_stream_read(bufs[i % ncopy], words, blocks)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        out.append({"bytes": nbytes, "copies": ncopy, "blocks": blocks, "us": round(us, 2),
                    "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)})
        del bufs, words
        torch.cuda.empty_cache()
    return out


def mfma_ceiling(torch, tq, dev):
    """int8 rate of tq_debug_mfma_ceiling (8 independent 32x32x32 MFMA chains per wave on register operands, no
    memory traffic): one and two blocks of 512 threads per compute unit, in TOP/s."""
    out = []
    iters = 256
    for per_cu in (1, 2):
        blocks = 256 * per_cu
        words = torch.empty(512 * blocks, dtype=torch.int32, device=dev)
        for _ in range(3):
            tq.tq_debug_mfma_ceiling(words, iters, blocks)
        torch.cuda.synchronize()
        steps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            tq.tq_debug_mfma_ceiling(words, iters, blocks)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        ops = 2.0 * 32 ** 3 * 8 * iters * blocks * 8  # 8 waves per block
        out.append({"blocks_per_cu": per_cu, "iters": iters, "us": round(us, 2),
                    "TOPs": round(ops / (us * 1e-6) / 1e12, 1), "frac_of_5000": round(ops / (us * 1e-6) / 5e15, 4)})
    return out


def activation_format(torch, tq, dev, steps=20):
    """The tile GEMM on the two activation-code formats, in us and TOP/s: nibble-packed codes (expanded in the loop
    like the weights) against one int8 byte per code (the layer's format), each with the integer-export epilogue
    (tq_debug_accumulate / tq_debug_accumulate_i8, int32 stores) and with the layer's dequantising bf16 epilogue
    without the low-rank term (tq_debug_gemm_w4a4).  Two code sets on 4096^3: the attention-projection workload's
    own codes (its X through tq_quantize_act, its weights through tq_pack_weight) and uniformly random codes."""
    from workloads import WORKLOADS, draw_linear

    wl = WORKLOADS["attn_proj"]
    n, k, m = wl.n, wl.d, wl.m
    c = draw_linear(wl, n=n)
    xp_w, sx_w = tq.tq_quantize_act(torch.from_numpy(c["X"]).to(dev).bfloat16(), 4)
    wp_w, sw_w = tq.tq_pack_weight(torch.from_numpy(c["R"]).to(dev), 4)
    del c
    g = torch.Generator(device=dev).manual_seed(5)

    def nibbles(codes):  # byte j: code 2 j in the low nibble, code 2 j + 1 in the high one
        codes = codes & 0xF
        return (codes[:, 0::2] | (codes[:, 1::2] << 4)).to(torch.uint8).contiguous()

    def codes_of(packed):  # nibble-packed -> int32 codes in [-8, 7]
        b = packed.to(torch.int32)
        lo, hi = b & 0xF, (b >> 4) & 0xF
        cds = torch.stack([lo, hi], dim=2).reshape(packed.shape[0], -1)
        return cds - 16 * (cds >= 8).to(torch.int32)

    def tile_order(codes):  # int8 bytes, within every 8 consecutive k the 4 even-k codes then the 4 odd-k codes
        g8 = codes.reshape(codes.shape[0], -1, 8)
        return torch.cat([g8[:, :, 0::2], g8[:, :, 1::2]], dim=2).reshape(codes.shape[0], -1).to(torch.int8).contiguous()

    cx = torch.randint(-8, 8, (n, k), dtype=torch.int32, device=dev, generator=g)
    cw = torch.randint(-8, 8, (m, k), dtype=torch.int32, device=dev, generator=g)
    sets = {"workload": (xp_w, tile_order(codes_of(xp_w)), wp_w, sx_w, sw_w),
            "random": (nibbles(cx), tile_order(cx), nibbles(cw), torch.rand(n, device=dev, generator=g) + 0.5,
                       torch.rand(m, device=dev, generator=g) * 0.01 + 0.001)}
    acc = torch.empty((n, m), dtype=torch.int32, device=dev)
    y = torch.empty((n, m), dtype=torch.bfloat16, device=dev)
    res = {"n": n, "k": k, "m": m}
    for sname, (xp, xi8, wp, sx, sw) in sets.items():
        runs = {"packed_int32": lambda: tq.tq_debug_accumulate(xp, wp, k, 4, acc=acc),
                "int8_int32": lambda: tq.tq_debug_accumulate_i8(xi8, wp, k, acc=acc),
                "packed_bf16_y": lambda: tq.tq_debug_gemm_w4a4(xp, True, sx, wp, sw, k, Y=y),
                "int8_bf16_y": lambda: tq.tq_debug_gemm_w4a4(xi8, False, sx, wp, sw, k, Y=y)}
        out = {}
        for name, fn in runs.items():
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            out[name] = {"us": round(us, 2), "TOPs": round(2.0 * n * k * m / (us * 1e-6) / 1e12, 1)}
            if name == "packed_int32":
                sums = acc.clone()
            elif name == "int8_int32":
                out["same_sums"] = bool(torch.equal(sums, acc))  # both formats give the same int32 sums
            elif name == "packed_bf16_y":
                y0 = y.clone()
            else:
                out["same_y"] = bool(torch.equal(y0, y))
        res[sname] = out
    return res


def cpu_baseline(wl, rows, seconds):
    """The oracle as it stands, timed on the host: the layer on the first `rows` tokens, repeated until about
    `seconds` of CPU work have been timed."""
    import oracle.tq_oracle as tqo
    from workloads import draw_linear

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    c = draw_linear(wl, n=rows)
    reps, dt = 0, 0.0
    while dt < seconds and reps < 100:
        t0 = time.perf_counter()
        tqo.tq_linear_ref(c["X"], c["R"], c["L1"], c["L2"])
        dt += time.perf_counter() - t0
        reps += 1
    ops = 2.0 * rows * wl.d * wl.m * reps
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": int(cores), "kind": "oracle",
            "sample": f"first {rows} of {wl.n} tokens, all {wl.m} output channels, {reps} repetitions; numpy/fp64 "
                      f"oracle incl. weight and activation quantisation, exact integer product, fp64 epilogue; "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="attn_proj")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--copies", type=int, default=16, help="weight copies cycled through (defeats the MALL)")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="tokens of the CPU oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time to accumulate (repetitions)")
    ap.add_argument("--n", type=int, default=0, help="tokens of the main workload (default: the workload's own)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only measure the streaming-read ceiling (tq_debug_stream_read) and print it")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only the int8 MFMA ceiling (tq_debug_mfma_ceiling), one JSON line")
    ap.add_argument("--activation-format", action="store_true",
                    help="only the tile GEMM on packed against int8 activation codes at 4096^3, one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (scales rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the layer's multi-GPU sharding is a "
              "design note, not a measured path", file=sys.stderr)
        sys.exit(2)

    import torch

    import rank_augmented_quantized_amd as tq
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}))
        return
    tq.load()
    if args.stream_ceiling:
        print(json.dumps({"stream_ceiling": stream_ceiling(torch, tq, dev, args.copies)}), flush=True)
        return
    if args.mfma_ceiling:
        print(json.dumps({"mfma_ceiling": mfma_ceiling(torch, tq, dev)}), flush=True)
        return
    if args.activation_format:
        print(json.dumps({"activation_format": activation_format(torch, tq, dev)}), flush=True)
        return
    wl = WORKLOADS[args.workload]
    n, d, m, r = args.n or wl.n, wl.d, wl.m, wl.r

    log(f"[bench] {wl.title} n={n}: building inputs")
    if wl.name == "two_subspace":  # the two-subspace layer (tq_linear_mp) on its own shape
        case = MpCase(wl, torch, tq, dev)
        n = wl.n
    else:
        case = LinearCase(wl, n, args.copies if n <= 256 else 2, torch, tq, dev)
    ms = time_calls(case, args.steps, args.warmup, torch)
    ops = 2.0 * n * d * m
    value = ops / (ms * 1e-3) / 1e12
    log(f"[bench] {wl.title}: {ms * 1e3:.1f} us/call, {value:.1f} TOPS")
    kms = kernel_ms(case, args.steps, torch, tq)
    gname = "gemm_w4a4" if "gemm_w4a4" in kms else max(kms, key=kms.get)
    gemm = kms[gname]
    achieved = ops / (gemm * 1e-3) / 1e12
    khash = kernel_source_hash()
    traffic = read_traffic(khash)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "frac": round(achieved / PEAK_INT8_TOPS, 4), "traffic": traffic if (gname == "gemm_w4a4" and wl.name == "attn_proj" and n == wl.n) else None,
                "kernel": gname,
                "kernel_us": round(gemm * 1e3, 2),
                "kernels_us": {k: round(v * 1e3, 2) for k, v in kms.items()}}
    log(f"[bench] kernels: {roofline['kernels_us']}")
    del case
    torch.cuda.empty_cache()

    sweep = []
    if not args.no_sweep:
        for name, ns in (("mlp_gate_up", (1, 16, 256, 4096)), ("mlp_down", (1, 8, 32)), ("small", (16,))):
            w = WORKLOADS[name]
            for nn in ns:
                c = LinearCase(w, nn, args.copies if nn <= 256 else 2, torch, tq, dev)
                t = time_calls(c, max(20, args.steps // 2), 10, torch)
                km = kernel_ms(c, 20, torch, tq)
                b = alg_bytes(nn, w.d, w.m, w.r, c.x_bytes)
                o = 2.0 * nn * w.d * w.m
                row = {"workload": w.title, "n": nn, "us": round(t * 1e3, 2), "TOPS": round(o / (t * 1e-3) / 1e12, 2),
                       "GBps": round(b / (t * 1e-3) / 1e9, 1), "pct_mfma": round(100 * o / (t * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
                       "pct_hbm": round(100 * b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                       "kernels_us": {k: round(v * 1e3, 2) for k, v in km.items()}}
                if nn <= 32:
                    tg = c.graph_ms(torch)
                    row.update({"graph_us": round(tg * 1e3, 2), "graph_GBps": round(b / (tg * 1e-3) / 1e9, 1),
                                "graph_pct_hbm": round(100 * b / (tg * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)})
                sweep.append(row)
                log(f"[bench] sweep {row}")
                del c
                torch.cuda.empty_cache()
        w = WORKLOADS["mlp_gate_up"]
        for nn in (1, 16, 4096):
            c = GroupCase(w, nn, 2, args.copies if nn <= 256 else 2, torch, tq, dev)
            steps = max(20, args.steps // 2)
            t = time_calls(c, steps, 10, torch)
            t_sep = time_calls(c.separate, steps, 10, torch)
            # X once; each layer's codes, scales, L1, L2 and its Y
            b = nn * w.d * 2 + 2 * (w.d * w.m // 2 + 4 * w.m + 2 * w.d * w.r + 2 * w.r * w.m + 2 * nn * w.m)
            o = 2.0 * nn * w.d * 2 * w.m
            row = {"workload": f"{w.title}: gate and up as one group", "n": nn, "us": round(t * 1e3, 2),
                   "separate_us": round(t_sep * 1e3, 2), "TOPS": round(o / (t * 1e-3) / 1e12, 2),
                   "GBps": round(b / (t * 1e-3) / 1e9, 1),
                   "pct_mfma": round(100 * o / (t * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
                   "pct_hbm": round(100 * b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
            sweep.append(row)
            log(f"[bench] sweep {row}")
            del c
            torch.cuda.empty_cache()
        for name, ns in (("attn_proj", (4096,)), ("mlp_gate_up", (1, 4096))):
            w = WORKLOADS[name]
            for nn in ns:
                c = QlrCase(w, nn, args.copies if nn <= 256 else 2, torch, tq, dev)
                t = time_calls(c, max(20, args.steps // 2), 10, torch)
                km = kernel_ms(c, 20, torch, tq)
                o = 2.0 * nn * w.d * w.m
                # X, the weight codes and scales, Q(U) and Q(V) with their scales (r padded to 32), Y
                rp = max(32, w.r)
                b = nn * w.d * 2 + w.d * w.m // 2 + 4 * w.m + rp * w.d // 2 + 4 * rp + w.m * rp // 2 + 4 * w.m + \
                    2 * nn * w.m
                row = {"workload": f"{w.title}: low-rank branch quantised too", "n": nn, "us": round(t * 1e3, 2),
                       "TOPS": round(o / (t * 1e-3) / 1e12, 2), "GBps": round(b / (t * 1e-3) / 1e9, 1),
                       "pct_mfma": round(100 * o / (t * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
                       "pct_hbm": round(100 * b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                       "kernels_us": {k: round(v * 1e3, 2) for k, v in km.items()}}
                sweep.append(row)
                log(f"[bench] sweep {row}")
                del c
                torch.cuda.empty_cache()
        for name, ns in (("attn_proj", (4096,)), ("mlp_gate_up", (16,))):
            w = WORKLOADS[name]
            for nn in ns:
                c = AsymCase(w, nn, args.copies if nn <= 256 else 2, torch, tq, dev)
                t = time_calls(c, max(20, args.steps // 2), 10, torch)
                km = kernel_ms(c, 20, torch, tq)
                o = 2.0 * nn * w.d * w.m
                b = alg_bytes(nn, w.d, w.m, w.r) + 4 * w.m
                row = {"workload": f"{w.title}: per-token asymmetric activations", "n": nn, "us": round(t * 1e3, 2),
                       "TOPS": round(o / (t * 1e-3) / 1e12, 2), "GBps": round(b / (t * 1e-3) / 1e9, 1),
                       "pct_mfma": round(100 * o / (t * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
                       "kernels_us": {k: round(v * 1e3, 2) for k, v in km.items()}}
                sweep.append(row)
                log(f"[bench] sweep {row}")
                del c
                torch.cuda.empty_cache()
        w = WORKLOADS["two_subspace"]
        from workloads import draw_two_subspace

        mp_inputs = draw_two_subspace(w)  # drawn once for the three lines
        for rht, asym, bits in ((False, False, (4, 8)), (True, False, (4, 8)), (False, True, (4, 8)),
                                (False, False, (3, 6))):
            log(f"[bench] {w.title}{' (rotation online)' if rht else ''}{' (asymmetric)' if asym else ''}"
                f"{' (6/3 bits)' if bits != (4, 8) else ''}: building inputs")
            c = MpCase(w, torch, tq, dev, rht=rht, asym=asym, case=mp_inputs, bits=bits)
            t = time_calls(c, 20, 3, torch)
            km = kernel_ms(c, 10, torch, tq)
            o = 2.0 * w.n * w.d * w.m
            b = w.n * w.d * 2 + (w.d - w.d_hi) * w.m // 2 + w.d_hi * w.m + 8 * w.m + 2 * w.n * w.m
            tag = ": unrotated X, rotation inside the quantiser" if rht else ""
            tag = ": per-token asymmetric activations" if asym else tag
            tag = ": 6-bit and 3-bit subspaces" if bits != (4, 8) else tag
            row = {"workload": w.title + tag, "n": w.n,
                   "us": round(t * 1e3, 2), "TOPS": round(o / (t * 1e-3) / 1e12, 2),
                   "GBps": round(b / (t * 1e-3) / 1e9, 1),
                   "pct_mfma": round(100 * o / (t * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
                   "kernels_us": {k: round(v * 1e3, 2) for k, v in km.items()}}
            sweep.append(row)
            log(f"[bench] sweep {row}")
            del c
            torch.cuda.empty_cache()

    ceiling = None if args.no_sweep else stream_ceiling(torch, tq, dev, args.copies)
    if ceiling:
        log(f"[bench] streaming-read ceiling {ceiling}")
    mceiling = None if args.no_sweep else mfma_ceiling(torch, tq, dev)
    if mceiling:
        log(f"[bench] int8 MFMA ceiling {mceiling}")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} tokens")
        cpu = cpu_baseline(wl, min(args.cpu_rows, n), args.cpu_seconds)
        log(f"[bench] cpu baseline {cpu}")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": wl.title, "n": n, "d": d, "m": m, "r": r, "x_dtype": wl.x_dtype, "y_dtype": "bf16",
                   "pct_int8_mfma_peak": round(100 * value / PEAK_INT8_TOPS, 2),
                   "why_this_workload": "the metric's prefill half (TOPS and % of int8 MFMA peak) is quoted on the "
                                        "4096-token attention projection, a whole single-GPU layer; the small case, "
                                        "the MLP sweep and the decode rows (GB/s and % of HBM) are the sweep lines"},
        "roofline": roofline, "cpu_baseline": cpu, "sweep": sweep, "stream_ceiling": ceiling, "mfma_ceiling": mceiling,
        "kernel_source_hash": khash,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Throughput of the quantized MoE grouped-GEMM path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload {0,1,...,9}] [--cold-steps C]
    python bench.py --peaks      (the chip's sustained HBM read rate and
                                  MFMA rate per dtype, measured on this GPU)

One step is one pass of the whole hot path over one batch of seeded
synthetic input already resident in HBM:
  0  W4A4 INT4, 64 tokens, E=4, top-2, K=N=256: route + INT4 GEMM + combine
  1  FP8 e4m3 1x128 / 128x128 block-scaled dense GEMM M=1024 N=4096
     K=7168: route (E=1) + FP8 GEMM
  2  NVFP4 W4A16 decode, 8 tokens, E=256, top-8, H=7168 I=2048:
     route + FC1 (SiLU-gated) + FC2 + combine; with --act f16 (default) the
     bf16 input is first cast to binary16 and h is binary16
  3  NVFP4 W4A16 prefill, 4096 tokens, Zipf(1.1) routing: as 2
  4  W4A4 INT4 Mixtral-like, 8192 tokens, E=8, top-2, H=4096 I=14336
     (default, the largest configuration): route + FC1 (SiLU-gated) + FC2
     (int4 rows in sorted order) + combine
  5  per-row INT4 quantization of 16384 fp16 rows of 14336 (the FC2 input
     of 4 in a full W4A4 chain)
  6  FP8 block-scaled MoE projection, decode: 8 tokens, E=256, top-8,
     N=4096 K=7168: route + FP8 GEMM (weight-streaming schedule)
  8  the complete W4A4 layer at 4's sizes from fp16 x: per-token int4 of
     x + FC1 (SiLU) + per-row int4 of h + FC2 + combine
  7  one-shot NVFP4 weight repack of 2's gate+up weights (E=256, 4096 rows,
     K=7168) from the up-first, 128x4-swizzled-scale layout of megamoe_rm.cu
  9  the W4A4 layer of 8 at one 8-token decode step (weight-streaming
     schedule)
Prints ONE JSON line: whole-path throughput (and the p10 / p50 / p90 of the
per-step times), the dominant kernel's roofline fraction (its launches timed
with HIP events on the launch stream inside the timed region) against the
published peak and against the peak measured on this GPU (--peaks, summarized
in profiles/peaks_mi355x.txt), and the CPU oracle's throughput on the host
as a reported baseline.  The steps run back to back with their inputs
resident; `cold_cache` adds C steps timed one by one after the caches were
evicted.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "grouped-GEMM TFLOP/s and weight GB/s per MI355X; % of MFMA / HBM roofline"
# MI355X published peaks (dense).
PEAK = {"hbm_GBps": 8000.0, "bf16": 2500.0, "fp8": 5000.0, "int8": 5000.0}


def _dev(x):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def _sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantized_moe_grouped_route_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_tag, sources):
    """HBM bytes per launch from the committed PMC summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256_16") != _sources_digest(sources):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- peaks
# MFMA kinds of the peak probe: (name, K per 32x32 instruction, published
# dense peak in T(FL)OP/s).
MFMA_KINDS = {0: ("int8", 32, 5000.0), 1: ("fp8", 64, 5000.0), 2: ("bf16", 16, 2500.0),
              3: ("fp16", 16, 2500.0), 4: ("fp6", 64, 10100.0), 5: ("fp4", 64, 10100.0)}
PEAKS_FILE = os.path.join(ROOT, "profiles", "peaks_mi355x.txt")


def measure_peaks(reps: int = 10):
    """The chip's sustained rates: HBM read (4 GiB streamed with 16-byte
    nontemporal loads into registers, and with nontemporal direct-to-LDS
    copies; the faster counts) and each MFMA kind on register operands (2
    workgroups of 4 waves per CU).  Median of `reps` launches timed with HIP
    events."""
    import ctypes as C
    import torch
    from quantized_moe_grouped_route_amd import build as b
    L = C.CDLL(b.PEAKS_LIB)
    L.moeq_peak_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_void_p]
    L.moeq_peak_read_lds.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p]
    L.moeq_peak_mfma.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream

    def timed(launch):
        ms = []
        for i in range(reps + 2):
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            assert launch() == 0
            z.record()
            torch.cuda.synchronize()
            if i >= 2:
                ms.append(a.elapsed_time(z))
        return float(np.median(ms))

    res = {}
    nbytes = 1 << 32
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    grid = cus * 8
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    ms = timed(lambda: L.moeq_peak_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, st))
    regs = dict(value=nbytes / (ms * 1e-3) / 1e9, unit="GB/s", spec=PEAK["hbm_GBps"], ms=ms)
    ms = timed(lambda: L.moeq_peak_read_lds(buf.data_ptr(), nbytes, cus * 2, st))
    lds = dict(value=nbytes / (ms * 1e-3) / 1e9, unit="GB/s", spec=PEAK["hbm_GBps"], ms=ms)
    # the bound is the faster way of streaming: register loads or LDS copies
    res["hbm_read"] = max(regs, lds, key=lambda r: r["value"])
    res["hbm_read_registers"] = regs
    res["hbm_read_lds_copies"] = lds
    del buf
    grid = cus * 2
    sinkf = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(0)
    for kind, (name, K, spec) in MFMA_KINDS.items():
        iters = 20000 if K == 16 else 10000
        src = torch.from_numpy(peak_operands(rng, name, grid * 256 * 64)).cuda()
        ms = timed(lambda: L.moeq_peak_mfma(kind, grid, iters, src.data_ptr(), sinkf.data_ptr(), st))
        ops = grid * 4 * iters * 4 * 2.0 * 32 * 32 * K
        res[name] = dict(value=ops / (ms * 1e-3) / 1e12, unit="TFLOP/s" if name != "int8" else "TOP/s",
                         spec=spec, ms=ms)
    return res


def peak_operands(rng, name, nbytes):
    """Operand bytes for the MFMA probe: finite values of the format, as the
    grouped GEMMs feed it (int8: nibbles times 16, as the INT4 GEMM splits
    them; fp8: e4m3 codes of N(0,1) values; bf16 / fp16: N(0,1); fp6 / fp4:
    uniform codes, all of which are finite)."""
    import torch
    n = nbytes
    if name == "int8":
        return ((rng.integers(-8, 8, n) * 16) & 0xFF).astype(np.uint8)
    if name == "fp8":
        x = torch.from_numpy(rng.standard_normal(n).astype(np.float32))
        return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if name in ("bf16", "fp16"):
        x = torch.from_numpy(rng.standard_normal(n // 2).astype(np.float32))
        return x.to(torch.bfloat16 if name == "bf16" else torch.float16).view(torch.uint8).numpy()
    return rng.integers(0, 256, n).astype(np.uint8)


def measured_peak(key):
    """The committed on-GPU measurement of one peak, or None."""
    if not os.path.exists(PEAKS_FILE):
        return None
    for line in open(PEAKS_FILE):
        if line.startswith(key + ":"):
            return float(line.split(":", 1)[1].split()[0])
    return None


# ---------------------------------------------------------------- workloads
class Workload:
    """Device buffers and the launch sequence of one step."""

    def __init__(self, idx: int, fc2: str = "sorted", act: str = "f16", sfl: str = "quads",
                 wl: str = "tiled"):
        import torch
        import synth
        import quantized_moe_grouped_route_amd as mq
        self.mq, self.idx, self.fc2, self.act, self.sfl, self.wl = mq, idx, fc2, act, sfl, wl
        self.cfg = synth.WORKLOADS[idx]
        self.d = d = synth.workload(idx)
        if self.cfg["kind"] == "repack":
            self._init_repack(torch)
            return
        if self.cfg["kind"] == "quant":
            self.E, self.k, self.T = 1, 1, self.cfg["rows"]
        else:
            self.E, self.k, self.T = d["E"], d["k"], d["T"]
        T, k, E = self.T, self.k, self.E
        P = T * k
        if self.cfg["kind"] == "quant":
            self._init_quant(torch)
            return
        self.ids = _dev(d["topk_ids"])
        self.tw = _dev(d["topk_weights"])
        i32 = dict(dtype=torch.int32, device="cuda")
        self.route_out = (torch.empty(E + 1, **i32), torch.empty(P, **i32), torch.empty(P, **i32),
                          torch.empty(1, **i32))
        nws = mq.route_workspace_bytes(T, k, E)
        self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
        kind = self.cfg["kind"]
        if kind == "int4chain":
            H, I = d["H"], d["I"]
            self.x = _dev(d["x"])
            self.w, self.sw = _dev(d["w"]), _dev(d["w_scale"])
            self.w2, self.sw2 = _dev(d["w2"]), _dev(d["w2_scale"])
            f16, u8, f32 = torch.float16, torch.uint8, torch.float32
            self.qx = torch.empty(T, H // 2, dtype=u8, device="cuda")
            self.sx = torch.empty(T, dtype=f32, device="cuda")
            self.h = torch.empty(P, I, dtype=f16, device="cuda")
            self.qh = torch.empty(P, I // 2, dtype=u8, device="cuda")
            self.sh = torch.empty(P, dtype=f32, device="cuda")
            self.y = torch.empty(P, H, dtype=f16, device="cuda")
            self.out = torch.empty(T, H, dtype=f16, device="cuda")
            self.flops = 2.0 * P * (2 * I * H + H * I)
            self.weight_bytes = None
            self.dtype = "int4_via_int8_mfma"
            self.dom = ("int4_prefill", ["gemm_int4.hip", "common.h", "tile.h"], "mfma", PEAK["int8"])
            if self.int4_streaming():  # weight GB/s against HBM
                self.active, self.fc1_bytes, self.weight_bytes = self.int4_stream_bytes()
                self.dom = ("int4_decode", ["gemm_int4.hip", "common.h", "tile.h", "pipeline.h"], "hbm",
                            PEAK["hbm_GBps"])
        elif kind == "fp8":
            self.a, self.sa = _dev(d["a"]), _dev(d["a_scale"])
            self.w, self.sw = _dev(d["w"]), _dev(d["w_scale"])
            self.y = torch.empty(P, d["N"], dtype=torch.bfloat16, device="cuda")
            self.flops = 2.0 * P * d["N"] * d["K"]
            ids = d["topk_ids"].reshape(-1)
            self.active = int(np.unique(ids[(ids >= 0) & (ids < E)]).size)
            self.weight_bytes = float(self.active * (d["N"] * d["K"] + (d["N"] // 128) * (d["K"] // 128) * 4))
            self.dtype = "fp8_e4m3"
            if idx == 6:
                self.dom = ("fp8_decode", ["gemm_fp8.hip", "common.h", "tile.h", "pipeline.h"], "hbm",
                            PEAK["hbm_GBps"])
            else:
                self.dom = ("fp8_prefill", ["gemm_fp8.hip", "common.h", "tile.h", "pipeline.h"], "mfma",
                            PEAK["fp8"])
        elif kind == "int4":
            self.a, self.sa = _dev(d["a"]), _dev(d["a_scale"])
            self.w, self.sw = _dev(d["w"]), _dev(d["w_scale"])
            self.dtype = "int4_via_int8_mfma"
            if idx == 0:
                self.y = torch.empty(P, d["N"], dtype=torch.float16, device="cuda")
                self.out = torch.empty(T, d["N"], dtype=torch.float16, device="cuda")
                self.flops = 2.0 * P * d["N"] * d["K"]
            else:
                I = d["N"] // 2
                self.h = torch.empty(P, I, dtype=torch.float16, device="cuda")
                self.a2, self.sa2 = _dev(d["a2"]), _dev(d["a2_scale"])
                self.w2, self.sw2 = _dev(d["w2"]), _dev(d["w2_scale"])
                self.y = torch.empty(P, d["N2"], dtype=torch.float16, device="cuda")
                self.out = torch.empty(T, d["N2"], dtype=torch.float16, device="cuda")
                self.flops = 2.0 * P * (d["N"] * d["K"] + d["N2"] * d["K2"])
            self.weight_bytes = None
            # the 64-token problem runs on the streaming schedule (its 256x256
            # tiles would occupy a handful of compute units)
            self.dom = (("int4_decode", ["gemm_int4.hip", "common.h", "tile.h", "pipeline.h"]) if idx == 0 else
                        ("int4_prefill", ["gemm_int4.hip", "common.h", "tile.h"])) + ("mfma", PEAK["int8"])
        else:  # nvfp4
            H, I = d["H"], d["I"]
            self.x = _dev(d["x"])
            # Scales in the library's K-quad-major layout by default: the seeded
            # bytes are iid, so they are read directly in that stored order.
            self.s1_host, self.s2_host = d["s1"], d["s2"]
            if sfl == "quads":
                self.s1_host = d["s1"].reshape(E, H // 64, 2 * I, 4)
                self.s2_host = d["s2"].reshape(E, I // 64, H, 4)
            # codes in the tiled layout by default: iid bytes, read in that order
            self.w1_host, self.w2_host = d["w1"], d["w2"]
            if wl == "tiled":
                self.w1_host = d["w1"].reshape(E, 2 * I // 16, H // 64, 16, 32)
                self.w2_host = d["w2"].reshape(E, H // 16, I // 64, 16, 32)
            self.w1, self.s1, self.g1 = _dev(self.w1_host), _dev(self.s1_host), _dev(d["g1"])
            self.w2, self.s2, self.g2 = _dev(self.w2_host), _dev(self.s2_host), _dev(d["g2"])
            hdt = torch.float16 if act == "f16" else torch.bfloat16
            self.xh = torch.empty(T, H, dtype=torch.float16, device="cuda") if act == "f16" else None
            self.h = torch.empty(P, I, dtype=hdt, device="cuda")
            self.y = torch.empty(P, H, dtype=torch.bfloat16, device="cuda")
            self.tw_flat = self.tw.reshape(-1)
            self.wq = mq.work_queue()  # tile balancing of the tiled schedule (one per stream)
            self.out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
            ids = d["topk_ids"].reshape(-1)
            valid = ids[(ids >= 0) & (ids < E)]
            self.active = int(np.unique(valid).size)
            per_expert = (2 * I * H // 2 + 2 * I * H // 16 + H * I // 2 + H * I // 16 + 8)
            self.weight_bytes = float(self.active * per_expert)
            self.fc1_bytes = float(self.active * (2 * I * H // 2 + 2 * I * H // 16 + 4))
            self.flops = 2.0 * valid.size * (2 * I * H + H * I)
            self.dtype = "f16_x_nvfp4" if act == "f16" else "bf16_x_nvfp4"
            if idx == 2:
                self.dom = ("nvfp4_decode", ["gemm_nvfp4.hip", "nvfp4.h", "common.h", "tile.h", "pipeline.h"], "hbm",
                            PEAK["hbm_GBps"])
            else:
                self.dom = ("nvfp4_prefill", ["gemm_nvfp4.hip", "nvfp4.h", "common.h", "tile.h", "pipeline.h"], "mfma",
                            PEAK["bf16"])

    def _init_quant(self, torch):
        rows, K = self.cfg["rows"], self.cfg["K"]
        self.x = _dev(self.d["x"])
        self.q = torch.empty(rows, K // 2, dtype=torch.uint8, device="cuda")
        self.qs = torch.empty(rows, dtype=torch.float32, device="cuda")
        self.weight_bytes = float(rows * (2 * K + K // 2 + 4))
        self.flops = 0.0
        self.dtype = "f16_to_int4"
        self.dom = ("quant_int4_rows_reg", ["quant.hip", "common.h"], "hbm", PEAK["hbm_GBps"])

    def _init_repack(self, torch):
        d = self.d
        self.E, self.k, self.T = d["E"], 1, 0
        self.w_in, self.sf_in = _dev(d["w"]), _dev(d["sf"])
        self.w_out = torch.empty_like(self.w_in)
        self.sf_out = torch.empty(d["E"], d["N"], d["K"] // 16, dtype=torch.uint8, device="cuda")
        self.weight_bytes = repack_bytes(d["E"], d["N"], d["K"])
        self.flops = 0.0
        self.dtype = "u8"
        self.dom = ("repack_nvfp4", ["repack.hip", "kernels.h", "common.h"], "hbm", PEAK["hbm_GBps"])

    def step(self, ev=None):
        """One pass of the path; `ev` = (start, end) events around the
        dominant kernel."""
        mq = self.mq
        kind = self.cfg["kind"]
        if kind == "quant":
            if ev: ev[0].record()
            mq.quantize_int4_rows(self.x, q=self.q, scale=self.qs)
            if ev: ev[1].record()
            return
        if kind == "repack":
            if ev: ev[0].record()
            mq.nvfp4_repack(self.w_in, self.sf_in, swap_halves=bool(self.cfg["swap"]), w_out=self.w_out,
                            sf_out=self.sf_out)
            if ev: ev[1].record()
            return
        offs, srt, p2s, _ = mq.moe_route_prep(self.ids, self.E, out=self.route_out, workspace=self.ws)
        if kind == "int4chain":
            mq.quantize_int4_rows(self.x, q=self.qx, scale=self.sx)
            if ev: ev[0].record()
            mq.grouped_gemm_qint4(self.qx, self.sx, self.w, self.sw, offs, srt, self.k, act="silu_mul",
                                  out=self.h)
            if ev: ev[1].record()
            mq.quantize_int4_rows(self.h, q=self.qh, scale=self.sh)
            mq.grouped_gemm_qint4(self.qh, self.sh, self.w2, self.sw2, offs, srt, self.k, a_row="sorted",
                                  out=self.y)
            mq.moe_scatter_combine(self.y, p2s, self.tw, out=self.out)
        elif kind == "fp8":
            if ev: ev[0].record()
            mq.grouped_gemm_qfp8_block(self.a, self.sa, self.w, self.sw, offs, srt, self.k, out=self.y)
            if ev: ev[1].record()
        elif kind == "int4" and self.idx == 0:
            if ev: ev[0].record()
            mq.grouped_gemm_qint4(self.a, self.sa, self.w, self.sw, offs, srt, self.k, out=self.y)
            if ev: ev[1].record()
            mq.moe_scatter_combine(self.y, p2s, self.tw, out=self.out)
        elif kind == "int4":
            import torch
            if ev: ev[0].record()
            mq.grouped_gemm_qint4(self.a, self.sa, self.w, self.sw, offs, srt, self.k, act="silu_mul",
                                  out=self.h)
            if ev: ev[1].record()
            mq.grouped_gemm_qint4(self.a2, self.sa2, self.w2, self.sw2, offs, srt, self.k,
                                  a_row="sorted", out=self.y)
            mq.moe_scatter_combine(self.y, p2s, self.tw, out=self.out)
        else:
            x = self.x
            if self.act == "f16":
                # megamoe_rm.cu's fp16 activations: the bf16 input is cast once
                x = mq.cast_bf16_to_f16(self.x, out=self.xh)
            if ev: ev[0].record()
            mq.grouped_gemm_qnvfp4(x, self.w1, self.s1, self.g1, offs, srt, self.k, act="silu_mul",
                                   out=self.h, out_dtype=self.h.dtype, work_queue=self.wq)
            if ev: ev[1].record()
            if self.fc2 == "pair":
                # top-k weight in FC2's epilogue, rows in pair order, then the pair sum
                mq.grouped_gemm_qnvfp4(self.h, self.w2, self.s2, self.g2, offs, srt, self.k,
                                       a_row="sorted", pair_weights=self.tw_flat, out=self.y,
                                       work_queue=self.wq)
                mq.moe_sum_pairs(self.y, p2s, self.T, self.k, out=self.out)
            else:
                mq.grouped_gemm_qnvfp4(self.h, self.w2, self.s2, self.g2, offs, srt, self.k,
                                       a_row="sorted", out=self.y, work_queue=self.wq)
                mq.moe_scatter_combine(self.y, p2s, self.tw, out=self.out)

    def dominant_launches(self):
        """(launches of the dominant kernel per step, index of the timed one)."""
        return (1, 0) if self.cfg["kind"] in ("fp8", "quant", "repack") or self.idx == 0 else (2, 0)

    def int4_streaming(self):
        """The W4A4 layer at decode size: few rows per expert, so the INT4
        GEMMs take the weight-streaming schedule."""
        return self.cfg["kind"] == "int4chain" and self.T * self.k < 16 * self.E

    def int4_stream_bytes(self):
        """(active experts, FC1 weight + scale bytes, FC1 + FC2 bytes) of the
        experts the step routes to."""
        d = self.d
        H, I, E = d["H"], d["I"], self.E
        ids = d["topk_ids"].reshape(-1)
        active = int(np.unique(ids[(ids >= 0) & (ids < E)]).size)
        fc1 = float(active * 2 * I * (H // 2 + 4))
        return active, fc1, fc1 + float(active * H * (I // 2 + 4))

    def dominant_bytes(self):
        """Fewest HBM bytes one launch of the dominant kernel can move: every
        operand read once, every output written once."""
        d, P = self.d, self.T * self.k
        kind = self.cfg["kind"]
        if kind in ("quant", "repack"):
            return self.weight_bytes
        if kind == "fp8":
            N, K = d["N"], d["K"]
            return float(P * K + self.weight_bytes + d["a_scale"].size * 4 + P * N * 2)
        if self.int4_streaming():
            return float(self.int4_stream_bytes()[1] + P * (d["H"] // 2 + 4) + P * d["I"] * 2)
        if kind in ("int4", "int4chain"):
            N, K = d["N"], d["K"]
            out = N * 2 if self.idx == 0 else N  # f16 y, or f16 h = N/2 columns
            return float(P * K // 2 + P * 4 + d["w"].size + d["w_scale"].size * 4 + P * out)
        H, I = d["H"], d["I"]
        return float(self.fc1_bytes + P * H * 2 + P * I * 2)

    def dominant_work(self):
        """Algorithmic work of one launch of the dominant kernel:
        (value, unit) in bytes (HBM-bound) or flops (MFMA-bound)."""
        d = self.d
        kind = self.cfg["kind"]
        if kind in ("quant", "repack"):
            return self.weight_bytes, "byte"
        if kind == "fp8" and self.idx == 6:
            return self.weight_bytes, "byte"
        if kind == "fp8":
            return 2.0 * self.T * self.k * d["N"] * d["K"], "flop"
        if self.int4_streaming():
            return self.int4_stream_bytes()[1], "byte"
        if kind in ("int4", "int4chain"):
            return 2.0 * self.T * self.k * d["N"] * d["K"], "flop"
        if self.idx == 2:
            return self.fc1_bytes, "byte"
        ids = d["topk_ids"].reshape(-1)
        return 2.0 * int(((ids >= 0) & (ids < self.E)).sum()) * 2 * d["I"] * d["H"], "flop"


def repack_bytes(E, N, K):
    """Bytes a repack must move: every weight and scale byte read once and
    written once."""
    return float(2 * E * N * (K // 2 + K // 16))


# ---------------------------------------------------------------- CPU oracle
def cpu_baseline(idx: int, d, budget_s: float = 10.0):
    """The CPU oracle, as it stands, on a bounded sample of the workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    kind = {0: "int4", 1: "fp8", 2: "nvfp4", 3: "nvfp4", 4: "int4", 5: "quant", 6: "fp8",
            7: "repack", 8: "int4", 9: "int4"}[idx]
    times = []
    if kind == "repack":
        ne = 64
        nbytes = repack_bytes(ne, d["N"], d["K"])
        while sum(times) < budget_s and len(times) < 5:
            t = time.perf_counter()
            oracle.repack_nvfp4(d["w"][:ne], d["sf"][:ne], True)
            times.append(time.perf_counter() - t)
        return dict(value=nbytes / float(np.median(times)) / 1e9, unit="GB/s", cores=cores, kind="oracle",
                    sample=f"{ne} of {d['E']} experts, median of {len(times)} runs")
    if kind == "quant":
        x = d["x"]
        rows = np.arange(0, x.shape[0], 64)
        nbytes = rows.size * (2 * x.shape[1] + x.shape[1] // 2 + 4)
        while sum(times) < budget_s and len(times) < 5:
            t = time.perf_counter()
            oracle.quantize_int4_rows(x[rows])
            times.append(time.perf_counter() - t)
        return dict(value=nbytes / float(np.median(times)) / 1e9, unit="GB/s", cores=cores, kind="oracle",
                    sample=f"{rows.size} of {x.shape[0]} rows, median of {len(times)} runs")
    off, srt, p2s, _ = oracle.route_prep(d["topk_ids"], d["E"])
    n = int(off[-1])
    if kind == "fp8" and idx == 6:
        # the rows of 4 active experts; weight GB/s over their bytes
        experts = [e for e in range(d["E"]) if off[e + 1] > off[e]][:4]
        rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
        nbytes = len(experts) * d["N"] * d["K"]
        while sum(times) < budget_s and len(times) < 5:
            t = time.perf_counter()
            oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                           d["k"], rows=rows)
            times.append(time.perf_counter() - t)
        return dict(value=nbytes / float(np.median(times)) / 1e9, unit="GB/s", cores=cores, kind="oracle",
                    sample=f"{rows.size} rows of {len(experts)} active experts, median of {len(times)} runs")
    if kind == "fp8":
        sample = "the whole workload (all rows)"
        work = 2.0 * n * d["N"] * d["K"]
        while sum(times) < budget_s and len(times) < 5:
            t = time.perf_counter()
            oracle.route_prep(d["topk_ids"], d["E"])
            oracle.grouped_gemm_qfp8_block(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                           d["k"])
            times.append(time.perf_counter() - t)
        return dict(value=work / float(np.median(times)) / 1e12, unit="TFLOP/s", cores=cores,
                    kind="oracle", sample=sample + f", median of {len(times)} runs")
    if kind == "int4" and idx == 9:
        # the FC1 rows of 2 active experts, on the oracle's own codes of x;
        # weight GB/s over those experts' bytes
        a, sa = oracle.quantize_int4_rows(d["x"])
        experts = [e for e in range(d["E"]) if off[e + 1] > off[e]][:2]
        rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
        nbytes = len(experts) * d["N"] * (d["K"] // 2 + 4)
        while sum(times) < budget_s and len(times) < 3:
            t = time.perf_counter()
            oracle.grouped_gemm_qint4(a, sa, "token", d["w"], d["w_scale"], off, srt, d["k"], act="silu_mul",
                                      rows=rows)
            times.append(time.perf_counter() - t)
        return dict(value=nbytes / float(np.median(times)) / 1e9, unit="GB/s", cores=cores, kind="oracle",
                    sample=f"{rows.size} rows of {len(experts)} active experts of FC1, median of {len(times)} runs")
    if kind == "int4":
        rows = np.arange(n) if idx == 0 else np.arange(0, n, max(1, n // 64))
        sample = "the whole workload" if idx == 0 else f"{rows.size} sorted rows of FC1 (gate+up, K={d['K']})"
        work = 2.0 * rows.size * d["N"] * d["K"]
        if idx == 8:                      # FC1 reads the oracle's own codes of x
            d = dict(d)
            d["a"], d["a_scale"] = oracle.quantize_int4_rows(d["x"])
        while sum(times) < budget_s and len(times) < 5:
            t = time.perf_counter()
            oracle.grouped_gemm_qint4(d["a"], d["a_scale"], "token", d["w"], d["w_scale"], off, srt,
                                      d["k"], act="none" if idx == 0 else "silu_mul", rows=rows)
            times.append(time.perf_counter() - t)
        return dict(value=work / float(np.median(times)) / 1e12, unit="TFLOP/s", cores=cores,
                    kind="oracle", sample=sample + f", median of {len(times)} runs")
    # nvfp4: the FC1 rows of a few experts; weight GB/s over the bytes read.
    H, I = d["H"], d["I"]
    experts = [e for e in range(d["E"]) if off[e + 1] > off[e]][:4]
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in experts])
    nbytes = len(experts) * (2 * I * H // 2 + 2 * I * H // 16)
    t = time.perf_counter()
    oracle.grouped_gemm_qnvfp4(d["x"], "token", d["w1"], d["s1"], d["g1"], off, srt, d["k"],
                               act="silu_mul", rows=rows)
    dt = time.perf_counter() - t
    if idx == 2:
        return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=cores, kind="oracle",
                    sample=f"FC1 of {len(experts)} active experts ({rows.size} rows)")
    return dict(value=2.0 * rows.size * 2 * I * H / dt / 1e12, unit="TFLOP/s", cores=cores,
                kind="oracle", sample=f"FC1 of {len(experts)} experts ({rows.size} rows)")


# ------------------------------------------------------- profile summaries
def profile_commands(idx: int, pdir: str):
    """The rocprofv3 runs whose outputs --summarize-profiles reduces."""
    run = f"python3 bench.py --workload {idx}"
    short = f"{run} --steps 3 --warmup 1 --cold-steps 0 --no-cpu-baseline"
    copy = "python3 bench.py --copy-calibration"
    pmc = "rocprofv3 --pmc {c} -d {d} -o run --output-format csv -- {r}"
    return {
        "trace": f"rocprofv3 --kernel-trace --stats -d {pdir}/trace_w{idx} -o run --output-format csv -- {run}",
        "fetch": pmc.format(c="FETCH_SIZE", d=f"{pdir}/fetch_w{idx}", r=short),
        "write": pmc.format(c="WRITE_SIZE", d=f"{pdir}/write_w{idx}", r=short),
        "copy_fetch": pmc.format(c="FETCH_SIZE", d=f"{pdir}/fetch_copy", r=copy),
        "copy_write": pmc.format(c="WRITE_SIZE", d=f"{pdir}/write_copy", r=copy),
        "counters": pmc.format(c=" ".join(COUNTERS), d=f"{pdir}/counters_w{idx}", r=short),
    }


# One rocprofv3 pass (at most 8 SQ and 2 GRBM counters): matrix-core busy
# cycles, the shader clock, and where the waves spend their time.
COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_WAVE_CYCLES", "SQ_WAIT_INST_ANY",
            "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE")
NOMINAL_GHZ = 2.4


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short_name(name):
    """Kernel base name: no return type, namespaces, template or call arguments."""
    base = name[5:] if name.startswith("void ") else name
    base = base.replace("(anonymous namespace)::", "").split("(")[0].split("<")[0]
    return base.split("::")[-1]


def summarize_profiles(idx: int, pdir: str, steps: int = 50, warmup: int = 10):
    """Reduce the rocprofv3 outputs of profile_commands() to the text
    summaries under profiles/: per-kernel duration statistics and, for the
    dominant kernel, HBM traffic per launch scaled by a copy of known size."""
    import synth
    cfg = synth.WORKLOADS[idx]
    wl = Workload.__new__(Workload)  # host-side fields only
    wl.idx, wl.cfg = idx, cfg
    if cfg["kind"] == "quant":
        wl.d = {}
        wl.T, wl.k, wl.E = cfg["rows"], 1, 1
        wl.weight_bytes = float(cfg["rows"] * (2 * cfg["K"] + cfg["K"] // 2 + 4))
    elif cfg["kind"] == "repack":
        wl.d = {}
        wl.T, wl.k, wl.E = 0, 1, cfg["E"]
        wl.weight_bytes = repack_bytes(cfg["E"], cfg["N"], cfg["K"])
    else:
        wl.d = synth.workload(idx)
        wl.T, wl.k, wl.E = wl.d["T"], wl.d["k"], wl.d["E"]
    d = wl.d
    tag = ("fp8_decode" if idx == 6 else None) or ("int4_decode" if idx in (0, 9) else None) or \
        {"fp8": "fp8_prefill", "int4": "int4_prefill", "int4chain": "int4_prefill", "quant": "quant_int4_rows_reg",
         "repack": "repack_nvfp4"}.get(cfg["kind"]) or \
        ("nvfp4_decode" if idx == 2 else "nvfp4_prefill")
    srcs = {"fp8_prefill": ["gemm_fp8.hip", "common.h", "tile.h", "pipeline.h"],
            "fp8_decode": ["gemm_fp8.hip", "common.h", "tile.h", "pipeline.h"],
            "int4_prefill": ["gemm_int4.hip", "common.h", "tile.h"],
            "int4_decode": ["gemm_int4.hip", "common.h", "tile.h", "pipeline.h"],
            "quant_int4_rows_reg": ["quant.hip", "common.h"],
            "repack_nvfp4": ["repack.hip", "kernels.h", "common.h"]}.get(
        tag, ["gemm_nvfp4.hip", "nvfp4.h", "common.h", "tile.h", "pipeline.h"])
    if cfg["kind"] == "fp8":
        ids = d["topk_ids"].reshape(-1)
        active = int(np.unique(ids[(ids >= 0) & (ids < wl.E)]).size)
        wl.weight_bytes = float(active * (d["N"] * d["K"] + (d["N"] // 128) * (d["K"] // 128) * 4))
    if cfg["kind"] == "nvfp4":
        H, I = d["H"], d["I"]
        ids = d["topk_ids"].reshape(-1)
        active = int(np.unique(ids[(ids >= 0) & (ids < wl.E)]).size)
        wl.fc1_bytes = float(active * (2 * I * H // 2 + 2 * I * H // 16 + 4))
    per_step, which = wl.dominant_launches()
    cmds = profile_commands(idx, pdir)

    def find(sub, suffix):
        path = os.path.join(pdir, sub, f"run_{suffix}.csv")
        if not os.path.exists(path):
            raise SystemExit(f"missing {path}: run the rocprofv3 commands first")
        return path

    def dominant(rows, key):
        rows = [r for r in rows if _short_name(r["Kernel_Name"]) == tag]
        rows.sort(key=lambda r: int(r[key]))
        return [r for i, r in enumerate(rows) if i % per_step == which]

    # durations: stats over all launches, the timed launches from the trace
    stats = _csv_rows(find(f"trace_w{idx}", "kernel_stats"))
    trace = dominant(_csv_rows(find(f"trace_w{idx}", "kernel_trace")), "Start_Timestamp")
    timed = trace[-steps:]
    dur_us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in timed]
    name = f"{tag}_{cfg['name']}"
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    lines = [f"# Kernel durations: {cfg['name']}", "",
             "Command (from the repository root, TMPDIR=/tmp):", "", f"    {cmds['trace']}", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {_short_name(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {r['Percentage']} |")
    lines += ["", f"Dominant kernel `{tag}`: launch {which + 1} of {per_step} per step, last {len(timed)} "
              f"launches of the trace (the timed steps): average {np.mean(dur_us):.2f} us, "
              f"min {np.min(dur_us):.2f}, max {np.max(dur_us):.2f}."]
    log = os.path.join(pdir, f"trace_w{idx}.log")
    if os.path.exists(log):
        for ln in open(log):
            if ln.startswith("{"):
                rec = json.loads(ln)
                lines += ["", f"bench.py line of the same run: kernel_ms {rec['roofline']['kernel_ms']} "
                          f"(HIP events), frac {rec['roofline']['frac']}, value {rec['value']} {rec['unit']}."]
    with open(os.path.join(ROOT, "profiles", f"{name}_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # traffic
    def counter(sub, ctr, rows_of):
        rows = [r for r in _csv_rows(find(sub, "counter_collection")) if r["Counter_Name"] == ctr]
        return [float(r["Counter_Value"]) for r in rows_of(rows)]
    copy_bytes = float((1 << 28) * 4)
    is_copy = lambda rows: [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
    cf = counter("fetch_copy", "FETCH_SIZE", is_copy)
    cw = counter("write_copy", "WRITE_SIZE", is_copy)
    f_fac = copy_bytes / (np.mean(cf) * 1024.0)
    w_fac = copy_bytes / (np.mean(cw) * 1024.0)
    dom = lambda rows: dominant(rows, "Dispatch_Id")
    fk = counter(f"fetch_w{idx}", "FETCH_SIZE", dom)
    wk = counter(f"write_w{idx}", "WRITE_SIZE", dom)
    fetch_b = float(np.mean(fk)) * 1024.0 * f_fac
    write_b = float(np.mean(wk)) * 1024.0 * w_fac
    alg = wl.dominant_bytes()
    txt = [f"kernel: {tag}", f"workload: {cfg['name']}",
           f"kernel_sources: {' '.join(srcs)}",
           f"kernel_sources_sha256_16: {_sources_digest(srcs)}",
           f"launches_counted: {len(fk)} (FETCH_SIZE), {len(wk)} (WRITE_SIZE); launch {which + 1} of "
           f"{per_step} per step",
           f"fetch_size_kib_per_launch: {np.mean(fk):.1f}",
           f"write_size_kib_per_launch: {np.mean(wk):.1f}",
           f"copy_calibration: 1 GiB device copy reads FETCH_SIZE {np.mean(cf):.1f} KiB, "
           f"WRITE_SIZE {np.mean(cw):.1f} KiB; factors fetch {f_fac:.4f}, write {w_fac:.4f}",
           f"fetch_bytes_per_launch: {fetch_b:.0f}",
           f"write_bytes_per_launch: {write_b:.0f}",
           f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
           f"algorithmic_bytes_per_launch: {alg:.0f}",
           f"traffic_over_algorithmic: {(fetch_b + write_b) / alg:.3f}",
           "commands (from the repository root, TMPDIR=/tmp):"]
    txt += [f"  {cmds[k]}" for k in ("fetch", "write", "copy_fetch", "copy_write")]
    with open(os.path.join(ROOT, "profiles", f"{name}_traffic.txt"), "w") as f:
        f.write("\n".join(txt) + "\n")
    print(f"wrote profiles/{name}_kernel_stats.md and profiles/{name}_traffic.txt")

    # counters (optional pass): matrix-core utilisation and clock of the
    # dominant kernel, per launch
    cdir = os.path.join(pdir, f"counters_w{idx}")
    if not os.path.isdir(cdir):
        return
    agent = [r for r in _csv_rows(find(f"counters_w{idx}", "agent_info")) if r.get("Name", "").startswith("gfx")][0]
    simds, xcc = int(agent["Simd_Count"]), int(agent["Num_Xcc"])
    by = {}
    for r in _csv_rows(find(f"counters_w{idx}", "counter_collection")):
        if _short_name(r["Kernel_Name"]) != tag:
            continue
        d = by.setdefault(int(r["Dispatch_Id"]), {"_r": r})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    disp = [by[k] for k in sorted(by)]
    disp = [d for i, d in enumerate(disp) if i % per_step == which]
    if not disp:
        raise SystemExit(f"no {tag} launches in {cdir}")

    def avg(key):
        return float(np.mean([d[key] for d in disp]))
    dur_s = float(np.mean([(int(d["_r"]["End_Timestamp"]) - int(d["_r"]["Start_Timestamp"])) * 1e-9 for d in disp]))
    gui = avg("GRBM_GUI_ACTIVE") / xcc          # shader cycles of one XCD over the launch
    busy = avg("SQ_VALU_MFMA_BUSY_CYCLES") / simds
    ctxt = [f"kernel: {tag}", f"workload: {cfg['name']}",
            f"kernel_sources: {' '.join(srcs)}",
            f"kernel_sources_sha256_16: {_sources_digest(srcs)}",
            f"launches_counted: {len(disp)}; launch {which + 1} of {per_step} per step",
            f"agent: {agent['Name']}, {simds} SIMDs, {xcc} XCDs",
            f"duration_us_per_launch: {dur_s * 1e6:.1f} (counter run)"]
    ctxt += [f"{k.lower()}_per_launch: {avg(k):.0f}" for k in COUNTERS]
    trace_s = float(np.mean(dur_us)) * 1e-6  # timed launches of the kernel-trace run
    ctxt += [f"duration_us_per_launch_kernel_trace: {trace_s * 1e6:.1f}",
             f"mfma_busy_cycles_per_simd: {busy:.0f}",
             f"mfma_busy_fraction_at_{NOMINAL_GHZ}ghz: {busy / (trace_s * NOMINAL_GHZ * 1e9):.3f} "
             f"(busy cycles per SIMD / (kernel-trace duration x nominal clock))",
             "GRBM_GUI_ACTIVE counts the whole counter window; the next two figures hold only where the "
             "launch is much longer than the counter run's dispatch overhead:"]
    if gui / dur_s / 1e9 > NOMINAL_GHZ or (trace_s < 200e-6 and dur_s > 1.1 * trace_s):
        # the counter window of a short launch takes in the dispatch around it
        why = (f"invalid for this launch (counter-run duration {dur_s * 1e6:.1f} us against "
               f"{trace_s * 1e6:.1f} us traced)")
        ctxt += [f"shader_clock_ghz: {why}", f"mfma_busy_fraction_of_active_cycles: {why}"]
    else:
        ctxt += [f"shader_clock_ghz: {gui / dur_s / 1e9:.3f} (GRBM_GUI_ACTIVE / XCDs / counter-run duration)",
                 f"mfma_busy_fraction_of_active_cycles: {busy / gui:.3f} "
                 f"(SQ_VALU_MFMA_BUSY_CYCLES / SIMDs / GRBM_GUI_ACTIVE per XCD)"]
    ctxt += [f"wave_time_waiting_fraction: {avg('SQ_WAIT_INST_ANY') / avg('SQ_WAVE_CYCLES'):.3f} "
             f"(SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)",
             f"wave_time_valu_fraction: {avg('SQ_ACTIVE_INST_VALU') / avg('SQ_WAVE_CYCLES'):.3f}",
             f"wave_time_lds_fraction: {avg('SQ_ACTIVE_INST_LDS') / avg('SQ_WAVE_CYCLES'):.3f}",
             "command (from the repository root, TMPDIR=/tmp):", f"  {cmds['counters']}"]
    with open(os.path.join(ROOT, "profiles", f"{name}_counters.txt"), "w") as f:
        f.write("\n".join(ctxt) + "\n")
    print(f"wrote profiles/{name}_counters.txt")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=4, choices=sorted(__import__("synth").WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed one by one after evicting the caches (a 1 GiB device read "
                         "between steps, outside each step's events), reported as cold_cache; "
                         "0 skips them")
    ap.add_argument("--act", choices=("bf16", "f16"), default="f16",
                    help="NVFP4 workloads: GEMMs on the bf16 activations, or on binary16 activations "
                         "(the bf16 input cast once, h kept in binary16; half the dequant work)")
    ap.add_argument("--sf-layout", choices=("rows", "quads"), default="quads",
                    help="NVFP4 workloads: block scales row-major [E][N][K/16] or K-quad-major "
                         "[E][K/64][N][4] (the library's layout for the tiled schedule)")
    ap.add_argument("--w-layout", choices=("rows", "tiled"), default="tiled",
                    help="NVFP4 workloads: E2M1 codes row-major [E][N][K/2] or tiled in 16-row x "
                         "64-K blocks (the library's layout for the tiled schedule)")
    ap.add_argument("--fc2", choices=("sorted", "pair"), default="sorted",
                    help="NVFP4 workloads: FC2 writes sorted rows and the combine applies the top-k "
                         "weights (sorted), or FC2's epilogue applies them and writes pair-ordered "
                         "rows that a pair sum adds (pair)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the sustained HBM read rate and each MFMA kind's rate on this "
                         "GPU, print them as the lines of profiles/peaks_mi355x.txt, and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 5 times (a kernel of known traffic "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--profile-commands", metavar="DIR",
                    help="print the rocprofv3 commands (outputs under DIR) that "
                         "--summarize-profiles reduces, one per line, and exit")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries of --workload from the rocprofv3 "
                         "outputs under DIR (host only) and exit")
    args = ap.parse_args()
    if args.profile_commands:
        print("\n".join(profile_commands(args.workload, args.profile_commands).values()))
        return
    if args.summarize_profiles:
        summarize_profiles(args.workload, args.summarize_profiles, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print("bench.py measures one MI355X: the path runs on a single GPU; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.peaks:
        res = measure_peaks()
        print(f"# Sustained peaks of one {torch.cuda.get_device_name(0)} "
              f"({torch.cuda.get_device_properties(0).multi_processor_count} CUs), median of 10 launches")
        print("# command (from the repository root): python3 bench.py --peaks")
        for k, v in res.items():
            print(f"{k}: {v['value']:.1f} {v['unit']} (published {v['spec']:.0f}, "
                  f"{v['value'] / v['spec']:.3f} of it; {v['ms']:.3f} ms per launch)")
        return
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": src.numel() * 4,
                          "copy_bytes_written_per_launch": dst.numel() * 4}), flush=True)
        return
    wl = Workload(args.workload, args.fc2, args.act, args.sf_layout, args.w_layout)
    torch.cuda.synchronize()
    host_s = []
    for _ in range(args.warmup):
        t = time.perf_counter()
        wl.step()
        host_s.append(time.perf_counter() - t)
    torch.cuda.synchronize()
    # The device must never wait for the host inside the timed region: a
    # bounded spin kernel holds the stream while the host enqueues every
    # timed step, so the events time the device's work, not the gaps of
    # the Python launches.  The spin ends before t0 is recorded.
    host_step_ms = 1e3 * float(np.median(host_s) if host_s else 1e-3)
    spin_ms = 2.0 + 1.5 * args.steps * host_step_ms
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(1 << 20)
    c1.record()
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 20) / max(c0.elapsed_time(c1), 1e-3)

    # Cold-cache steps, before the timed region so that a trace's last K
    # launches are still the timed ones.  Each step follows a 1 GiB device
    # read, which evicts the L2s and the 256 MB Infinity Cache (a read, so no
    # dirty lines are written back during the step), then a spin that holds
    # the stream while the host enqueues the step; its events open after both.
    cold = None
    if args.cold_steps > 0:
        flush_src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        flush_dst = torch.empty((), dtype=torch.float32, device="cuda")
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.cold_steps)]
        for a, z in cev:
            torch.sum(flush_src, dim=None, out=flush_dst)
            torch.cuda._sleep(int((0.2 + 2.0 * host_step_ms) * cycles_per_ms))
            a.record()
            wl.step()
            z.record()
        torch.cuda.synchronize()
        cold_ms = np.array([a.elapsed_time(z) for a, z in cev])
        del flush_src, flush_dst

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    # The timed region runs from `first` to `last`.  Per-step times come from
    # the events that open each step's dominant launch: step i spans one
    # period, from evs[i][0] to evs[i + 1][0] (K - 1 periods).  Each event
    # record costs the stream about 3 us, so no separate step marks are
    # recorded.
    first, last = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(min(spin_ms, 2000.0) * cycles_per_ms))
    wall = time.perf_counter()
    first.record()
    for i in range(args.steps):
        wl.step(evs[i])
    last.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    ms = first.elapsed_time(last) / args.steps
    step_ms = np.array([evs[i][0].elapsed_time(evs[i + 1][0]) for i in range(args.steps - 1)]
                       if args.steps > 1 else [ms])
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    cfg = wl.cfg
    if args.workload in (2, 5, 6, 7, 9):
        rate, unit = (lambda t: wl.weight_bytes / (t * 1e-3) / 1e9), "GB/s"
    else:
        rate, unit = (lambda t: wl.flops / (t * 1e-3) / 1e12), "TFLOP/s"
    value = rate(ms)
    if args.cold_steps > 0:
        c50 = float(np.percentile(cold_ms, 50))
        cold = {"steps": args.cold_steps,
                "ms_per_step_p10_p50_p90": [round(float(np.percentile(cold_ms, q)), 5) for q in (10, 50, 90)],
                "value_at_p50": round(rate(c50), 3), "unit": unit,
                "flush": "1 GiB device read before each step, outside the step's events"}
    work, wunit = wl.dominant_work()
    tag, srcs, bound, peak = wl.dom
    if wunit == "byte":
        achieved, runit = work / (dom_ms * 1e-3) / 1e9, "GB/s"
    else:
        achieved, runit = work / (dom_ms * 1e-3) / 1e12, "TFLOP/s"
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": runit,
            "frac": round(achieved / peak, 4), "traffic": _traffic(f"{tag}_{cfg['name']}", srcs),
            "kernel": tag, "kernel_ms": round(dom_ms, 5)}
    mkey = {"hbm": "hbm_read"}.get(bound) or {"int4_via_int8_mfma": "int8", "fp8_e4m3": "fp8",
                                              "f16_x_nvfp4": "fp16", "bf16_x_nvfp4": "bf16"}.get(wl.dtype)
    mpeak = measured_peak(mkey) if mkey else None
    if mpeak:
        roof["peak_measured"] = round(mpeak, 1)
        roof["frac_of_measured"] = round(achieved / mpeak, 4)
    config = {"workload": cfg["name"]}
    config.update({k: v for k, v in cfg.items() if k not in ("name", "kind")})
    if cfg["kind"] == "nvfp4":
        config["fc2_epilogue"] = args.fc2
        config["activations"] = args.act
        config["scale_layout"] = args.sf_layout
        config["code_layout"] = args.w_layout
    if args.workload in (2, 6, 9):
        config["active_experts"] = wl.active
        config["weight_bytes"] = wl.weight_bytes
    rec = {"metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "ms_per_step_p10_p50_p90": [round(float(np.percentile(step_ms, q)), 5) for q in (10, 50, 90)],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
           "data": "synthetic (seeded generators, shapes of the workload)", "config": config,
           "roofline": roof}
    if cold:
        rec["cold_cache"] = cold
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.workload, wl.d)
    rec["host_wall_s_incl_spin"] = round(wall, 4)
    rec["host_enqueue_ms_per_step"] = round(1e3 * float(np.median(host_s)) if host_s else 0.0, 4)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

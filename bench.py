"""Throughput of the quantized MoE grouped-GEMM path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload {0,1,2,3,4}]

One step is one pass of the whole hot path over one batch of seeded
synthetic input already resident in HBM:
  0  W4A4 INT4, 64 tokens, E=4, top-2, K=N=256: route + INT4 GEMM + combine
  1  FP8 e4m3 1x128 / 128x128 block-scaled dense GEMM M=1024 N=4096
     K=7168 (default): route (E=1) + FP8 GEMM
  2  NVFP4 W4A16 decode, 8 tokens, E=256, top-8, H=7168 I=2048:
     route + FC1 (SiLU-gated) + FC2 + combine
  3  NVFP4 W4A16 prefill, 4096 tokens, Zipf(1.1) routing: as 2
  4  W4A4 INT4 Mixtral-like, 8192 tokens, E=8, top-2, H=4096 I=14336:
     route + FC1 (SiLU-gated) + FC2 (int4 rows in sorted order) + combine
Prints ONE JSON line: whole-path throughput, the dominant kernel's roofline
fraction (its launches timed with HIP events on the launch stream inside the
timed region) and the CPU oracle's throughput on the host as a reported
baseline.
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


# ---------------------------------------------------------------- workloads
class Workload:
    """Device buffers and the launch sequence of one step."""

    def __init__(self, idx: int):
        import torch
        import synth
        import quantized_moe_grouped_route_amd as mq
        self.mq, self.idx = mq, idx
        self.cfg = synth.WORKLOADS[idx]
        self.d = d = synth.workload(idx)
        self.E, self.k, self.T = d["E"], d["k"], d["T"]
        T, k, E = self.T, self.k, self.E
        P = T * k
        self.ids = _dev(d["topk_ids"])
        self.tw = _dev(d["topk_weights"])
        i32 = dict(dtype=torch.int32, device="cuda")
        self.route_out = (torch.empty(E + 1, **i32), torch.empty(P, **i32), torch.empty(P, **i32),
                          torch.empty(1, **i32))
        nws = mq.route_workspace_bytes(T, k, E)
        self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
        kind = self.cfg["kind"]
        if kind == "fp8":
            self.a, self.sa = _dev(d["a"]), _dev(d["a_scale"])
            self.w, self.sw = _dev(d["w"]), _dev(d["w_scale"])
            self.y = torch.empty(P, d["N"], dtype=torch.bfloat16, device="cuda")
            self.flops = 2.0 * P * d["N"] * d["K"]
            self.weight_bytes = float(self.w.numel() + self.sw.numel() * 4)
            self.dtype = "fp8_e4m3"
            self.dom = ("fp8_prefill", ["gemm_fp8.hip", "common.h", "tile.h"], "mfma", PEAK["fp8"])
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
            self.dom = ("int4_prefill", ["gemm_int4.hip", "common.h", "tile.h"], "mfma", PEAK["int8"])
        else:  # nvfp4
            H, I = d["H"], d["I"]
            self.x = _dev(d["x"])
            self.w1, self.s1, self.g1 = _dev(d["w1"]), _dev(d["s1"]), _dev(d["g1"])
            self.w2, self.s2, self.g2 = _dev(d["w2"]), _dev(d["s2"]), _dev(d["g2"])
            self.h = torch.empty(P, I, dtype=torch.bfloat16, device="cuda")
            self.y = torch.empty(P, H, dtype=torch.bfloat16, device="cuda")
            self.out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
            ids = d["topk_ids"].reshape(-1)
            valid = ids[(ids >= 0) & (ids < E)]
            self.active = int(np.unique(valid).size)
            per_expert = (2 * I * H // 2 + 2 * I * H // 16 + H * I // 2 + H * I // 16 + 8)
            self.weight_bytes = float(self.active * per_expert)
            self.fc1_bytes = float(self.active * (2 * I * H // 2 + 2 * I * H // 16 + 4))
            self.flops = 2.0 * valid.size * (2 * I * H + H * I)
            self.dtype = "bf16_x_nvfp4"
            if idx == 2:
                self.dom = ("nvfp4_decode", ["gemm_nvfp4.hip", "nvfp4.h", "common.h", "tile.h"], "hbm",
                            PEAK["hbm_GBps"])
            else:
                self.dom = ("nvfp4_prefill", ["gemm_nvfp4.hip", "nvfp4.h", "common.h", "tile.h"], "mfma",
                            PEAK["bf16"])

    def step(self, ev=None):
        """One pass of the path; `ev` = (start, end) events around the
        dominant kernel."""
        mq = self.mq
        offs, srt, p2s, _ = mq.moe_route_prep(self.ids, self.E, out=self.route_out, workspace=self.ws)
        kind = self.cfg["kind"]
        if kind == "fp8":
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
            if ev: ev[0].record()
            mq.grouped_gemm_qnvfp4(self.x, self.w1, self.s1, self.g1, offs, srt, self.k, act="silu_mul",
                                   out=self.h)
            if ev: ev[1].record()
            mq.grouped_gemm_qnvfp4(self.h, self.w2, self.s2, self.g2, offs, srt, self.k,
                                   a_row="sorted", out=self.y)
            mq.moe_scatter_combine(self.y, p2s, self.tw, out=self.out)

    def dominant_work(self):
        """Algorithmic work of one launch of the dominant kernel:
        (value, unit) in bytes (HBM-bound) or flops (MFMA-bound)."""
        d = self.d
        kind = self.cfg["kind"]
        if kind == "fp8":
            return 2.0 * self.T * self.k * d["N"] * d["K"], "flop"
        if kind == "int4":
            return 2.0 * self.T * self.k * d["N"] * d["K"], "flop"
        if self.idx == 2:
            return self.fc1_bytes, "byte"
        ids = d["topk_ids"].reshape(-1)
        return 2.0 * int(((ids >= 0) & (ids < self.E)).sum()) * 2 * d["I"] * d["H"], "flop"


# ---------------------------------------------------------------- CPU oracle
def cpu_baseline(idx: int, d, budget_s: float = 10.0):
    """The CPU oracle, as it stands, on a bounded sample of the workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    kind = {0: "int4", 1: "fp8", 2: "nvfp4", 3: "nvfp4", 4: "int4"}[idx]
    off, srt, p2s, _ = oracle.route_prep(d["topk_ids"], d["E"])
    n = int(off[-1])
    times = []
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
    if kind == "int4":
        rows = np.arange(n) if idx == 0 else np.arange(0, n, max(1, n // 64))
        sample = "the whole workload" if idx == 0 else f"{rows.size} sorted rows of FC1 (gate+up, K={d['K']})"
        work = 2.0 * rows.size * d["N"] * d["K"]
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=1, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device-to-device 5 times (a kernel of known traffic "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one MI355X: the path runs on a single GPU; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": src.numel() * 4,
                          "copy_bytes_written_per_launch": dst.numel() * 4}), flush=True)
        return
    wl = Workload(args.workload)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall = time.perf_counter()
    t0.record()
    for i in range(args.steps):
        wl.step(evs[i])
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    ms = t0.elapsed_time(t1) / args.steps
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    cfg = wl.cfg
    if args.workload == 2:
        value, unit = wl.weight_bytes / (ms * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = wl.flops / (ms * 1e-3) / 1e12, "TFLOP/s"
    work, wunit = wl.dominant_work()
    tag, srcs, bound, peak = wl.dom
    if wunit == "byte":
        achieved, runit = work / (dom_ms * 1e-3) / 1e9, "GB/s"
    else:
        achieved, runit = work / (dom_ms * 1e-3) / 1e12, "TFLOP/s"
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": runit,
            "frac": round(achieved / peak, 4), "traffic": _traffic(f"{tag}_{cfg['name']}", srcs),
            "kernel": tag, "kernel_ms": round(dom_ms, 5)}
    config = {"workload": cfg["name"]}
    config.update({k: v for k, v in cfg.items() if k not in ("name", "kind")})
    if args.workload == 2:
        config["active_experts"] = wl.active
        config["weight_bytes"] = wl.weight_bytes
    rec = {"metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
           "data": "synthetic (seeded generators, shapes of the workload)", "config": config,
           "roofline": roof}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(args.workload, wl.d)
    rec["host_wall_s_timed"] = round(wall, 4)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

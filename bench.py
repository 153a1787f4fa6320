#!/usr/bin/env python3
"""Forward-pass throughput of the ternary-expert MoE block on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--sweep FILE]

A step is one forward pass of the whole block (router + delta, top-k, grouping,
gate/up, down, combine + correction) over one batch of synthetic tokens, with
every input already resident in HBM.  Each step uses the next of R copies of
the layer's expert banks (R chosen so the copies exceed 1 GB, more than the
256 MB Infinity Cache) and the next of P activation sets, so routing changes
from step to step and weights come from HBM.

Prints one JSON line: whole-job tokens/s, the roofline of the dominant kernel
(the gate/up expert kernel) from the library's stage events inside the timed
region, and the fp64 oracle timed on the host on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-block tokens/s (decode b=1..64, prefill 4k) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16

# name -> (layer config, tokens, mode)
WORKLOADS = {
    "olmoe-b1": ("olmoe", 1, "decode"), "olmoe-b8": ("olmoe", 8, "decode"),
    "olmoe-b64": ("olmoe", 64, "decode"),
    "a3b35-b1": ("a3b35", 1, "decode"), "a3b35-b8": ("a3b35", 8, "decode"),
    "a3b35-b32": ("a3b35", 32, "decode"), "a3b35-p4096": ("a3b35", 4096, "prefill"),
    "flashnext-b1": ("flashnext", 1, "decode"), "flashnext-b8": ("flashnext", 8, "decode"),
    "flashnext-b64": ("flashnext", 64, "decode"), "flashnext-p4096": ("flashnext", 4096, "prefill"),
    "skewed-p16384": ("skewed", 16384, "prefill"),
    # the router delta and the correction as ternary PQ2_0 containers
    "olmoe-b1-q": ("olmoe", 1, "decode", "q"), "a3b35-b1-q": ("a3b35", 1, "decode", "q"),
    "flashnext-b1-q": ("flashnext", 1, "decode", "q"), "flashnext-b64-q": ("flashnext", 64, "decode", "q"),
    "a3b35-p4096-q": ("a3b35", 4096, "prefill", "q"),
    # the router delta as rank-512 fp16 factors U V (the FlashNext release's form)
    "flashnext-b1-fd": ("flashnext", 1, "decode", "fd"), "flashnext-b64-fd": ("flashnext", 64, "decode", "fd"),
    "flashnext-p4096-fd": ("flashnext", 4096, "prefill", "fd"),
}
DELTA_FACTOR_RANK = 512
# the line the default run prints: the Flash-Next-shaped layer (the largest
# configuration) at prefill 4096, with its decode b = 64 and the skewed
# 16384-token prefill carried in the same record
DEFAULT_WORKLOAD = "flashnext-p4096"
EXTRA_WORKLOADS = ("flashnext-b64", "skewed-p16384")
# the ternary quantizer (bfloat16 weights -> containers) on every expert bank of a
# layer: name -> (layer config, container id, rule 0 absmean / 1 Lloyd)
QUANT_WORKLOADS = {
    "quant-lloyd-a3b35": ("a3b35", 142, 1),
    "quant-absmean-a3b35": ("a3b35", 142, 0),
    "quant-lloyd-flashnext": ("flashnext", 143, 1),
}
# the Q4_0 n-gram table gather: name -> (tokens, rows per token)
PLE_WORKLOADS = {"ple-b64": (64, 48), "ple-p4096": (4096, 48)}
PLE_ROWS, PLE_ROW_LEN = 320_001_536, 160
PLE_METRIC = "Q4_0 n-gram table rows gathered and decoded per second"
# the k=1 draft head: name -> (tokens, hidden h, inner m); 2048 x 4096 is the card's 50 MB
MTP_WORKLOADS = {"mtp-b1": (1, 2048, 4096), "mtp-b64": (64, 2048, 4096)}
MTP_METRIC = "k=1 draft head evaluations (tokens) per second"
# the rank-r branch on its own (as on the attention output): name -> (tokens, d, r, ternary A and B)
LOWRANK_WORKLOADS = {"lowrank-b1": (1, 2048, 512, False), "lowrank-b64": (64, 2048, 512, False),
                     "lowrank-p4096": (4096, 2048, 512, False), "lowrank-b1-q": (1, 2048, 512, True)}
LOWRANK_METRIC = "rank-r branch applications y + B(A x) (tokens) per second"
QUANT_METRIC = "ternary quantizer weights/s (bf16 -> PQ2_0 / PTQ1_0, absmean or Lloyd g128)"
# VALU lane operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
ALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# algorithmic lane operations per weight: the absmean step (|w|, the group sum,
# the code compare) and each Lloyd round (code compare, masked sum, count)
QUANT_OPS_ABSMEAN, QUANT_OPS_ROUND = 3, 3
DESCR = {
    "olmoe": "OLMoE-shaped MoE block (d=2048, 64 PQ2_0 experts, ffn 1024, top-8, rank-512 correction)",
    "a3b35": "35B-A3B-class MoE block (d=2048, 128 PQ2_0 experts, ffn 768, top-8, rank-512 correction)",
    "flashnext": "Flash-Next-shaped MoE block (d=3072, 512 PTQ1_0 experts top-10 + 1 shared, ffn 512, "
                 "rank-512 correction)",
    "skewed": "Skewed-routing stress at Flash-Next shape (Zipf 1.1 popularity, mixed PQ2_0/PTQ1_0, "
              "1% x50 outliers)",
}


EXPERT_SOURCES = ("device_common.h", "moe_experts.hip", "moe_internal.h")
QUANT_SOURCES = ("device_common.h", "moe_quant.hip", "wave_ops.h")
PLE_SOURCES = ("device_common.h", "moe_ple.hip")
MTP_SOURCES = ("device_common.h", "dense_rows.h", "moe_kernels.hip", "moe_internal.h", "moe_mtp.hip")
LOWRANK_SOURCES = ("device_common.h", "dense_rows.h", "moe_dense.hip", "moe_kernels.hip", "moe_internal.h")


def kernel_source_hash(names=EXPERT_SOURCES) -> str:
    """Hash of the sources a kernel is compiled from (by default the expert
    gate/up and down kernels)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "ternary_quantized_moe_amd", "csrc")
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, sources=EXPERT_SOURCES):
    """Measured HBM traffic of the dominant kernel (profiles/traffic.json), or
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("src_sha") != kernel_source_hash(sources):
        return None
    return rec.get("traffic_bytes_per_launch")


def f16_bits_of(dtype, factors):
    """fp16 bits of the product U V of two fp16-bit factor matrices."""
    import numpy as np
    u, v = [np.ascontiguousarray(a).view(np.float16).astype(dtype) for a in factors]
    return (u @ v).astype(np.float16).view(np.uint16)


def f16_expansion(trits, scale_bits):
    """fp16 bits of s * t for trits [rows, cols] and scale bits [rows, cols/128]:
    the scale with its sign flipped for t = -1, +0 for t = 0."""
    import numpy as np
    rows, cols = trits.shape
    s = np.repeat(scale_bits.astype(np.uint32), 128, axis=1).reshape(rows, cols)
    bits = np.where(trits < 0, s ^ 0x8000, s)
    return np.where(trits == 0, 0, bits).astype(np.uint16)


class Bench:
    def __init__(self, workload: str):
        import numpy as np
        import torch

        import ternary_quantized_moe_amd as tq
        from synthetic import CONFIGS, LayerGen

        self.np, self.torch, self.tq = np, torch, tq
        self.workload = workload
        cname, self.T, self.mode = WORKLOADS[workload][:3]
        variant = WORKLOADS[workload][3] if len(WORKLOADS[workload]) > 3 else ""
        self.ternary_corr, self.factored = variant == "q", variant == "fd"
        self.cfg = c = CONFIGS[cname]
        self.gen = g = LayerGen(c)
        self.formats = g.formats()
        dev = self.dev = torch.device("cuda:0")
        t0 = time.time()
        data, offsets = tq.build_banks(self.source, c.n_banks, self.formats, c.d_model, c.d_ff)
        self.offsets = offsets
        self.bank_bytes = int(data.size)
        base = torch.from_numpy(data).to(dev)
        self.R = max(1, math.ceil(1.0e9 / self.bank_bytes))
        self.banks = [tq.ExpertBanks.from_tensors(base if i == 0 else base.clone(), offsets, self.formats,
                                                  c.d_model, c.d_ff, c.n_experts, c.n_shared)
                      for i in range(self.R)]
        self.gu_bytes = np.where(self.formats == 142, 34, 28).astype(np.int64) * 2 * c.d_ff * c.d_model // 128
        self.dn_bytes = self.gu_bytes // 2
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
        self.router_bits = g.router_bits()
        self.router = t(self.router_bits)
        if self.ternary_corr:
            # PQ2_0 containers packed by the library; the oracle and the CPU
            # baseline get their exact fp16 expansions s * t
            parts = [g.delta_q_parts(), g.corr_a_q_parts(), g.corr_b_q_parts()]
            self.delta, self.corr_a, self.corr_b = [
                torch.from_numpy(tq.pack(142, tr.reshape(-1), sb.reshape(-1))).to(dev) for tr, sb in parts]
            self.delta_bits, self.a_bits, self.b_bits = [f16_expansion(tr, sb) for tr, sb in parts]
            self.delta_factors = None
        elif self.factored:
            self.delta_factors = g.delta_factor_bits(DELTA_FACTOR_RANK)
            self.du, self.dv = [t(a) for a in self.delta_factors]
            self.delta_bits = self.delta = None
            self.a_bits, self.b_bits = g.corr_a_bits(), g.corr_b_bits()
            self.corr_a, self.corr_b = t(self.a_bits), t(self.b_bits)
        else:
            self.delta_factors = None
            self.delta_bits = g.delta_bits()
            self.a_bits, self.b_bits = g.corr_a_bits(), g.corr_b_bits()
            self.delta = t(self.delta_bits)
            self.corr_a, self.corr_b = t(self.a_bits), t(self.b_bits)
        self.P = 16 if self.mode == "decode" else 2
        self.x_bits = [g.tokens(self.T, p) for p in range(self.P)]
        self.x = [t(xb) for xb in self.x_bits]
        self.y = torch.empty_like(self.x[0])
        if self.factored:
            need = tq.lib().moe_workspace_bytes_factored(self.banks[0].c, self.T, c.top_k, c.rank, DELTA_FACTOR_RANK)
            # the routing of the sets below takes U V rounded to fp16 as a dense
            # delta: it stands in for the factored choice (touched banks, bytes)
            uv = f16_bits_of(np.float64, self.delta_factors)
        else:
            need = tq.workspace_bytes(self.banks[0], self.T, c.top_k, c.rank)
            uv = self.delta_bits
        self.ws = tq.alloc_workspace(need, dev)
        # realised routing of every activation set (untimed): touched banks, slots
        self.touched, self.idx = [], []
        for p in range(self.P):
            r = tq.route(self.x[p], self.router, t(uv), c.n_experts, c.top_k)
            counts = r["counts"].cpu().numpy()
            touched = np.nonzero(counts)[0]
            self.touched.append(np.concatenate([touched, np.arange(c.n_experts, c.n_banks)]))
            self.idx.append(r["idx"].cpu().numpy())
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0

    def source(self, e):
        return self.gen.expert_trits(e), self.gen.expert_scales(e)

    def step(self, i: int):
        c = self.cfg
        if self.factored:
            self.tq.forward_factored(self.x[i % self.P], self.router, self.du, self.dv, self.banks[i % self.R],
                                     self.corr_a, self.corr_b, c.top_k, y=self.y, workspace=self.ws)
        elif self.ternary_corr:
            self.tq.forward_q(self.x[i % self.P], self.router, self.delta, self.banks[i % self.R], self.corr_a,
                              self.corr_b, c.rank, c.top_k, y=self.y, workspace=self.ws)
        else:
            self.tq.forward(self.x[i % self.P], self.router, self.delta, self.banks[i % self.R], self.corr_a,
                            self.corr_b, c.top_k, y=self.y, workspace=self.ws)

    # ---- parity before timing ----------------------------------------------------
    def parity(self, n_tokens: int = 4) -> float:
        np = self.np
        from oracle import moe as omoe
        c = self.cfg
        self.step(0)
        self.torch.cuda.synchronize()
        y = self.y.cpu().numpy().view(np.uint16)
        T = self.T
        toks = np.unique(np.linspace(0, T - 1, min(n_tokens, T)).astype(int))
        ob = omoe.LazyBanks(self.source, self.formats, c.d_model, c.d_ff, c.n_experts, c.n_shared)
        # (with factors, the oracle's own top-k: the device's choice is not exported)
        ref = omoe.forward(self.x_bits[0][toks], self.router_bits, self.delta_bits, ob, self.a_bits,
                           self.b_bits, c.top_k, forced_idx=None if self.factored else self.idx[0][toks],
                           delta_factors=self.delta_factors)
        yg = omoe.bf16_to_f64(y[toks])
        return float((np.abs(yg - ref.y).max(axis=1) / np.linalg.norm(ref.y, axis=1)).max())

    # ---- algorithmic work ----------------------------------------------------------
    def alg(self, p: int):
        """(whole-block bytes, gate/up bytes, whole-block flops, gate/up flops) of one
        step on activation set p, from its realised routing."""
        c = self.cfg
        T, d, f, E, r, k, S = self.T, c.d_model, c.d_ff, c.n_experts, c.rank, c.top_k, c.n_shared
        touched = self.touched[p]
        n_pos = T * k + S * T
        expert_bytes = int((self.gu_bytes[touched] + self.dn_bytes[touched]).sum())
        dense_bytes = 34 / 128 if self.ternary_corr else 2       # per weight of the delta, A and B
        delta_w = E * d if not self.factored else DELTA_FACTOR_RANK * (E + d)
        block_bytes = int(expert_bytes + 2 * E * d + dense_bytes * (delta_w + 2 * r * d) + 4 * T * d)
        gu_bytes = int(self.gu_bytes[touched].sum()) + 2 * T * d + 2 * n_pos * f
        block_flops = 2 * (n_pos * 3 * d * f + T * E * d + 2 * T * r * d)
        if self.factored:
            block_flops += 2 * T * DELTA_FACTOR_RANK * (d + E)
        gu_flops = 2 * n_pos * 2 * f * d
        return block_bytes, gu_bytes, block_flops, gu_flops


HOST = {}


def host_cpu():
    """The host CPU as lscpu reports it (model, physical cores = cores per
    socket x sockets) and the CPUs this process may run on.  Called before the
    GPU is touched: it starts lscpu as a child process."""
    if HOST:
        return HOST
    import subprocess
    model, phys = None, None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
        kv = {}
        for line in out.splitlines():
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        model = kv.get("Model name")
        phys = int(kv.get("Core(s) per socket", "0")) * int(kv.get("Socket(s)", "0")) or None
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    HOST.update({"cpu_model": model or "unknown", "physical_cores": phys, "cpus_available": avail})
    return HOST


def cpu_baseline(b: Bench, budget_s: float = 4.0, runs: int = 3):
    """The fp64 oracle, as it stands, on the first s tokens of activation set 0:
    the median of `runs` passes with BLAS threads = the physical cores this
    process may use, and the median of `runs` single-threaded passes."""
    np = b.np
    from oracle import codec, moe as omoe
    from threadpoolctl import threadpool_limits
    c = b.cfg
    host = host_cpu()
    threads = min(host["physical_cores"] or host["cpus_available"], host["cpus_available"])
    x = omoe.bf16_to_f64(b.x_bits[0])
    w = omoe.f16_to_f64(b.router_bits) + (omoe.factored_delta(*b.delta_factors) if b.factored
                                          else omoe.f16_to_f64(b.delta_bits))
    order = np.argsort(-(x @ w.T), axis=1, kind="stable")[:, :c.top_k]

    def needed(s):
        return sorted(set(order[:s].reshape(-1).tolist()) | set(range(c.n_experts, c.n_banks)))

    # cost of one bank decode (untimed probe)
    probe = omoe.LazyBanks(b.source, b.formats, c.d_model, c.d_ff, c.n_experts, c.n_shared)
    blob = probe.container(0)
    t0 = time.perf_counter()
    codec.decode(int(b.formats[0]), blob, 3 * c.d_model * c.d_ff)
    per_bank = time.perf_counter() - t0
    s = min(b.T, 64)
    while s > 1 and len(needed(s)) * per_bank > budget_s:
        s //= 2
    banks_needed = needed(s)
    # pre-pack (untimed) the banks the sample touches with the oracle codec
    offsets = np.zeros(c.n_banks, dtype=np.int64)
    chunks, pos = [], 0
    for e in banks_needed:
        blob = probe.container(e)
        offsets[e] = pos
        chunks.append(blob)
        pos += blob.size
    banks = omoe.Banks(np.concatenate(chunks), offsets, b.formats, c.d_model, c.d_ff, c.n_experts,
                       c.n_shared)

    def passes(n_threads):
        times = []
        with threadpool_limits(n_threads):
            for _ in range(runs):
                t0 = time.perf_counter()
                omoe.forward(b.x_bits[0][:s], b.router_bits, b.delta_bits, banks, b.a_bits, b.b_bits, c.top_k,
                             delta_factors=b.delta_factors)
                times.append(time.perf_counter() - t0)
        return times

    multi, single = passes(threads), passes(1)
    med, med1 = float(np.median(multi)), float(np.median(single))
    return {"value": s / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {s} of {b.T} tokens of activation set 0 ({len(banks_needed)} expert banks "
                      f"decoded per pass from the packed bytes); median of {runs} passes",
            "times_s": [round(t, 3) for t in multi],
            "single_thread": {"value": s / med1, "unit": "tokens/s", "cores": 1,
                              "times_s": [round(t, 3) for t in single]},
            "host": dict(host)}


def run(workload: str, steps: int, warmup: int, with_cpu: bool = True):
    import numpy as np
    import torch
    import ternary_quantized_moe_amd as tq

    b = Bench(workload)
    c = b.cfg
    warm = tq.StageTimer(max(warmup, 1), stages=[2])
    for i in range(warmup):
        with warm.step():
            b.step(i)
    torch.cuda.synchronize()
    # timed region: the K steps, with events around the dominant kernel on every
    # `every`-th step (an event record costs a few microseconds of stream time,
    # which is noise in a prefill step but not in a decode step)
    every = 4 if b.mode == "decode" else 1
    timer = tq.StageTimer((steps + every - 1) // every, stages=[2])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % every == 0:
            with timer.step():
                b.step(warmup + i)
        else:
            b.step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gu_ms = timer.ms()[2]
    # per-stage breakdown in a separate pass (every stage bracketed by events)
    n_brk = min(steps, 20)
    brk = tq.StageTimer(n_brk)
    for i in range(n_brk):
        with brk.step():
            b.step(i)
    stage_ms = brk.ms()

    # the oracle spot check comes after the timing: on a fresh machine, the first
    # heavy numpy work left the host busy for seconds and slowed the launches
    par = b.parity()
    works = [b.alg((warmup + i) % b.P) for i in range(steps)]
    block_bytes = float(np.mean([w[0] for w in works]))
    sampled = [w for i, w in enumerate(works) if i % every == 0]  # the steps the events timed
    gu_bytes = float(np.mean([w[1] for w in sampled]))
    block_flops = float(np.mean([w[2] for w in works]))
    gu_flops = float(np.mean([w[3] for w in sampled]))
    ms_step = elapsed * 1e3 / steps
    gu_s = gu_ms * 1e-3
    if b.mode == "decode":
        ach = gu_bytes / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": load_traffic(workload),
                "kernel": "expert_kernel<gate/up>", "alg_bytes_per_launch": int(gu_bytes),
                "avg_launch_us": round(gu_s * 1e6, 2), "timed_steps_with_events": f"1 in {every}"}
        block = {"alg_bytes": int(block_bytes), "achieved_GBs": round(block_bytes / (ms_step * 1e-3) / 1e9, 1),
                 "hbm_frac": round(block_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    else:
        ach = gu_flops / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": load_traffic(workload),
                "kernel": "expert_kernel<gate/up>", "alg_flops_per_launch": int(gu_flops),
                "avg_launch_us": round(gu_s * 1e6, 2), "timed_steps_with_events": f"1 in {every}"}
        block = {"alg_flops": int(block_flops),
                 "achieved_TFLOPs": round(block_flops / (ms_step * 1e-3) / 1e12, 1),
                 "mfma_frac": round(block_flops / (ms_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
    rec = {
        "metric": METRIC,
        "value": round(steps * b.T / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{DESCR[c.name]}, {b.mode} {b.T} tokens"
                               + (", router delta and correction as ternary PQ2_0 containers" if b.ternary_corr else "")
                               + (f", router delta as rank-{DELTA_FACTOR_RANK} fp16 factors" if b.factored else ""),
                   "name": workload,
                   "tokens": b.T, "mode": b.mode, "bank_replicas": b.R, "activation_sets": b.P,
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "block": block,
        "stages_ms": {n: round(float(v), 4) for n, v in zip(tq.STAGES, stage_ms)},
        "stages_note": "per-stage means from a separate pass with every stage bracketed by events",
        "parity_max_row_err": par,
    }
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(b)
    del b
    torch.cuda.empty_cache()
    return rec


# --------------------------------------------------------------------------- quantizer
def quant_shape(workload: str):
    from synthetic import CONFIGS
    cname, fmt, method = QUANT_WORKLOADS[workload]
    c = CONFIGS[cname]
    return c, fmt, method, c.n_banks * 3 * c.d_ff, c.d_model


def quant_cpu_baseline(fmt, method, d_w, out, rounds, budget_groups=65536):
    """The oracle quantizer, as it stands, on the first groups of the input; its
    containers and rounds are compared with the device's for the same groups."""
    import numpy as np
    from oracle import codec, quant
    G = min(budget_groups if method == 1 else 16 * budget_groups, d_w.numel() // 128)
    w = d_w.view(-1)[:G * 128].cpu().numpy().view(np.uint16)
    reps, dt = 0, 0.0
    while dt < 10.0 and (reps == 0 or dt * (reps + 1) / reps < 30.0):
        t0 = time.perf_counter()
        t, sb, _, r = quant.quantize_groups(w, method)
        data = codec.pack(fmt, t, sb)
        dt += time.perf_counter() - t0
        reps += 1
    bb = codec.block_bytes(fmt)
    got = out[:G * bb].cpu().numpy().reshape(G, bb)
    bad = int(np.count_nonzero(np.any(got != data.reshape(G, bb), axis=1)))
    bad_rounds = int(np.count_nonzero(rounds[:G].cpu().numpy() != r))
    # numpy's elementwise work runs on one thread (no BLAS call in the quantizer)
    base = {"value": reps * G * 128 / dt, "unit": "weights/s", "cores": 1, "kind": "oracle",
            "sample": f"first {G} of {d_w.numel() // 128} groups, {reps} pass(es), {dt:.1f} s"}
    return base, {"groups_checked": G, "groups_differing": bad, "rounds_differing": bad_rounds}


def run_quant(workload: str, steps: int, warmup: int, with_cpu: bool = True):
    import torch
    import ternary_quantized_moe_amd as tq
    from synthetic.weights import weights_bf16_device

    c, fmt, method, rows, cols = quant_shape(workload)
    n = rows * cols
    groups = n // 128
    bb = 34 if fmt == 142 else 28
    t0 = time.time()
    d_w = weights_bf16_device(rows, cols, seed=0).view(-1)
    out = torch.empty(groups * bb, dtype=torch.uint8, device="cuda:0")
    rounds = torch.empty(groups, dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    for _ in range(warmup):
        tq.quantize_device(fmt, method, d_w, out=out)
    torch.cuda.synchronize()
    # one kernel launch per step, bracketed by events on the launch stream
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        tq.quantize_device(fmt, method, d_w, out=out, stream=stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_s = sum(a.elapsed_time(b) for a, b in ev) / steps * 1e-3
    # the rounds per group (untimed; the same input gives the same rounds)
    tq.quantize_device(fmt, method, d_w, out=out, rounds=rounds)
    mean_rounds = float(rounds.to(torch.float64).mean().item())
    alg_bytes = 2 * n + groups * bb
    alg_ops = n * (QUANT_OPS_ABSMEAN + QUANT_OPS_ROUND * mean_rounds)
    hbm = alg_bytes / launch_s / 1e9
    ops = alg_ops / launch_s / 1e12
    src = QUANT_SOURCES
    if method == 0:
        roof = {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(hbm / HBM_PEAK_GBS, 4), "traffic": load_traffic(workload, src)}
    else:
        roof = {"bound": "alu", "achieved": round(ops, 2), "peak": round(ALU_PEAK_TOPS, 2), "unit": "TOP/s",
                "frac": round(ops / ALU_PEAK_TOPS, 4), "traffic": load_traffic(workload, src),
                "hbm_GBs": round(hbm, 1), "hbm_frac": round(hbm / HBM_PEAK_GBS, 4)}
    roof.update({"kernel": "quantize_kernel", "alg_bytes_per_launch": int(alg_bytes),
                 "alg_ops_per_launch": int(alg_ops), "mean_lloyd_rounds": round(mean_rounds, 4),
                 "avg_launch_us": round(launch_s * 1e6, 2)})
    rule = "Lloyd" if method == 1 else "absmean"
    rec = {
        "metric": QUANT_METRIC,
        "value": round(steps * n / elapsed, 1),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{rule} ternary quantizer into {'PQ2_0' if fmt == 142 else 'PTQ1_0'} over every "
                               f"expert bank of the {DESCR[c.name]}: {n} bfloat16 weights ({groups} groups)",
                   "name": workload, "weights": n, "parallelism": "single-gpu", "setup_s": round(setup_s, 1)},
        "roofline": roof,
    }
    if with_cpu:
        print(f"{workload}: timed, {launch_s * 1e3:.3f} ms per launch; oracle on the host next",
              file=sys.stderr, flush=True)
        rec["cpu_baseline"], rec["parity"] = quant_cpu_baseline(fmt, method, d_w, out, rounds)
    del d_w, out, rounds
    torch.cuda.empty_cache()
    return rec


# --------------------------------------------------------------------------- n-gram table
def ple_cpu_baseline(d_table, d_idx, out, budget_rows=4096):
    """The oracle row decode, as it stands, on the first rows of the row list;
    its rows are compared with the device's."""
    import numpy as np
    import torch
    from oracle import ple
    n = min(budget_rows, d_idx.numel())
    rows = d_idx[:n]
    sub = d_table[rows].cpu().numpy()                 # the sample's table rows, in list order
    reps, dt = 0, 0.0
    while dt < 10.0 and (reps == 0 or dt * (reps + 1) / reps < 30.0):
        t0 = time.perf_counter()
        want = ple.gather(sub, n, PLE_ROW_LEN, np.arange(n))
        dt += time.perf_counter() - t0
        reps += 1
    got = out[:n].cpu().numpy().astype(np.float64)
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    # one thread: a Python loop over rows and blocks
    base = {"value": reps * n / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n} of {d_idx.numel()} rows of the list, {reps} pass(es), {dt:.1f} s"}
    return base, {"rows_checked": n, "rows_differing": int(np.count_nonzero(~same.all(axis=1)))}


def run_ple(workload: str, steps: int, warmup: int, with_cpu: bool = True):
    import torch
    import ternary_quantized_moe_amd as tq
    from synthetic.ple import q4_table_device, row_list_device

    tokens, per_token = PLE_WORKLOADS[workload]
    n_idx = tokens * per_token
    t0 = time.time()
    d_table = q4_table_device(PLE_ROWS, PLE_ROW_LEN, seed=0)
    # P row lists, one per step in turn, so each step reads other rows
    P = 16 if tokens <= 64 else 4
    lists = [row_list_device(n_idx, PLE_ROWS, seed=p) for p in range(P)]
    out = torch.empty((n_idx, PLE_ROW_LEN), dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    for i in range(warmup):
        tq.ple_gather(d_table, PLE_ROWS, PLE_ROW_LEN, lists[i % P], out=out)
    stream = torch.cuda.current_stream()
    # events around one launch in four for small row lists (a record costs host
    # time comparable to the launch), around every launch otherwise
    every = 4 if tokens <= 256 else 1
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range((steps + every - 1) // every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % every == 0:
            ev[i // every][0].record(stream)
            tq.ple_gather(d_table, PLE_ROWS, PLE_ROW_LEN, lists[i % P], out=out, stream=stream)
            ev[i // every][1].record(stream)
        else:
            tq.ple_gather(d_table, PLE_ROWS, PLE_ROW_LEN, lists[i % P], out=out, stream=stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_s = sum(a.elapsed_time(b) for a, b in ev) / len(ev) * 1e-3
    row_bytes = PLE_ROW_LEN // 32 * 18
    alg_bytes = n_idx * (8 + row_bytes + 4 * PLE_ROW_LEN)       # index, Q4_0 row, fp32 row
    hbm = alg_bytes / launch_s / 1e9
    rec = {
        "metric": PLE_METRIC,
        "value": round(steps * n_idx / elapsed, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(elapsed * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"gather and decode of {n_idx} rows ({tokens} tokens x {per_token} rows) of a "
                               f"Q4_0 n-gram table of {PLE_ROWS} rows x {PLE_ROW_LEN} values "
                               f"({PLE_ROWS * row_bytes / 1e9:.1f} GB, rows uniform at random) into fp32",
                   "name": workload, "rows": n_idx, "row_lists": P, "parallelism": "single-gpu",
                   "setup_s": round(setup_s, 1)},
        "roofline": {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(hbm / HBM_PEAK_GBS, 4), "traffic": load_traffic(workload, PLE_SOURCES),
                     "kernel": "ple_gather_kernel", "alg_bytes_per_launch": int(alg_bytes),
                     "avg_launch_us": round(launch_s * 1e6, 2), "timed_steps_with_events": f"1 in {every}"},
    }
    if with_cpu:
        print(f"{workload}: timed, {launch_s * 1e6:.1f} us per launch; oracle on the host next",
              file=sys.stderr, flush=True)
        rec["cpu_baseline"], rec["parity"] = ple_cpu_baseline(d_table, lists[0], out if P == 1 else
                                                              tq.ple_gather(d_table, PLE_ROWS, PLE_ROW_LEN,
                                                                            lists[0]))
    del d_table, lists, out
    torch.cuda.empty_cache()
    return rec


# --------------------------------------------------------------------------- draft head
def mtp_cpu_baseline(hid, emb, w, got_bits):
    """The oracle head, as it stands, on every token of the batch; its rows are
    compared with the device's."""
    import numpy as np
    from oracle import moe as omoe, mtp
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    reps, dt = 0, 0.0
    while dt < 10.0 and (reps == 0 or dt * (reps + 1) / reps < 30.0):
        t0 = time.perf_counter()
        ref = mtp.head(hid, emb, *w)
        dt += time.perf_counter() - t0
        reps += 1
    got = omoe.bf16_to_f64(got_bits)
    err = float((np.abs(got - ref).max(axis=1) / np.linalg.norm(ref, axis=1)).max())
    T = hid.shape[0]
    return ({"value": reps * T / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
             "sample": f"all {T} tokens, {reps} pass(es), {dt:.1f} s"}, err)


def run_mtp(workload: str, steps: int, warmup: int, with_cpu: bool = True):
    import numpy as np
    import torch
    import ternary_quantized_moe_amd as tq
    from synthetic.mtp import head_inputs, head_weights

    T, h, m = MTP_WORKLOADS[workload]
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    t0 = time.time()
    w = head_weights(h, m, 0)
    # R copies of the weights, so each step reads them from HBM (over the 256 MB Infinity Cache)
    per_copy = 2 * (m * 2 * h + h * m)
    R = max(1, math.ceil(1.0e9 / per_copy))
    copies = [[t(a) for a in w] for _ in range(R)]
    P = 16
    inputs = [head_inputs(T, h, p) for p in range(P)]
    dev_in = [(t(a), t(b)) for a, b in inputs]
    y = torch.empty((T, h), dtype=torch.int16, device=dev)
    ws = tq.alloc_workspace(tq.lib().moe_draft_head_workspace_bytes(T, h, m), dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step(i):
        w1, b1, w2, b2 = copies[i % R]
        hid, emb = dev_in[i % P]
        tq.draft_head(hid, emb, w1, b1, w2, b2, y=y, workspace=ws)

    # the warmup uses every weight copy once before the timed steps
    for i in range(max(warmup, R)):
        step(i)
    torch.cuda.synchronize()
    # events bracket fc1's product (the library's stage events 0 and 1)
    every = 4 if T <= 256 else 1      # events on one step in four at decode sizes
    timer = tq.StageTimer((steps + every - 1) // every, stages=[0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % every == 0:
            with timer.step():
                step(warmup + i)
        else:
            step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fc1_s = timer.ms()[0] * 1e-3
    splits = 1 if T > 256 else 8
    fc1_bytes = 2 * m * 2 * h + 2 * T * 2 * h + 4 * T * m          # weights, input, fp32 product
    head_bytes = 2 * (m * 2 * h + h * m) + 2 * (m + h) + 2 * T * 2 * h + 2 * T * h
    ach = fc1_bytes / fc1_s / 1e9
    ms_step = elapsed * 1e3 / steps
    rec = {
        "metric": MTP_METRIC,
        "value": round(steps * T / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"k=1 draft head fc1 [{m} x {2 * h}] / gelu / fc2 [{h} x {m}] in fp16 "
                               f"({per_copy / 1e6:.1f} MB of weights), {T} token(s) per evaluation",
                   "name": workload, "tokens": T, "weight_replicas": R, "input_sets": P,
                   "parallelism": "single-gpu", "setup_s": round(setup_s, 1)},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": load_traffic(workload, MTP_SOURCES),
                     "kernel": ("xproj_split_kernel (fc1)" if T <= 32 else "xproj_wide_kernel (fc1)") if T <= 256
                     else "dense_gemm_kernel (fc1)",
                     "alg_bytes_per_launch": int(fc1_bytes), "avg_launch_us": round(fc1_s * 1e6, 2),
                     "k_slices": splits, "timed_steps_with_events": f"1 in {every}"},
        "head": {"alg_bytes": int(head_bytes),
                 "achieved_GBs": round(head_bytes / (ms_step * 1e-3) / 1e9, 1),
                 "hbm_frac": round(head_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if with_cpu:
        step(0)
        torch.cuda.synchronize()
        got = y.cpu().numpy().view(np.uint16)
        print(f"{workload}: timed, {ms_step * 1e3:.1f} us per step; oracle on the host next", file=sys.stderr,
              flush=True)
        rec["cpu_baseline"], rec["parity_max_row_err"] = mtp_cpu_baseline(*inputs[0], w, got)
    del copies, dev_in
    torch.cuda.empty_cache()
    return rec


# --------------------------------------------------------------------------- low-rank branch
def lowrank_cpu_baseline(x, yin, a, b, got_bits):
    """The oracle's y + B (A x), as it stands, on every token of the batch; its
    rows are compared with the device's."""
    import numpy as np
    from oracle import moe as omoe
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    reps, dt = 0, 0.0
    while dt < 10.0 and (reps == 0 or dt * (reps + 1) / reps < 30.0):
        t0 = time.perf_counter()
        ref = omoe.lowrank_apply(x, yin, a, b)
        dt += time.perf_counter() - t0
        reps += 1
    got = omoe.bf16_to_f64(got_bits)
    err = float((np.abs(got - ref).max(axis=1) / np.linalg.norm(ref, axis=1)).max())
    T = x.shape[0]
    return ({"value": reps * T / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
             "sample": f"all {T} tokens, {reps} pass(es), {dt:.1f} s"}, err)


def run_lowrank(workload: str, steps: int, warmup: int, with_cpu: bool = True):
    import numpy as np
    import torch
    import ternary_quantized_moe_amd as tq
    from synthetic import CONFIGS, LayerGen

    T, d, r, ternary = LOWRANK_WORKLOADS[workload]
    dev = torch.device("cuda:0")
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    t0 = time.time()
    g = LayerGen(CONFIGS["a3b35"])        # d = 2048, rank 512
    assert (g.cfg.d_model, g.cfg.rank) == (d, r)
    if ternary:
        (ta, sa), (tb, sb) = g.corr_a_q_parts(), g.corr_b_q_parts()
        qa, qb = tq.pack(142, ta.reshape(-1), sa.reshape(-1)), tq.pack(142, tb.reshape(-1), sb.reshape(-1))
        a_bits, b_bits = f16_expansion(ta, sa), f16_expansion(tb, sb)
        per_copy = qa.nbytes + qb.nbytes
        mk = lambda: (None, torch.from_numpy(qa).to(dev), None, torch.from_numpy(qb).to(dev))
    else:
        a_bits, b_bits = g.corr_a_bits(), g.corr_b_bits()
        per_copy = 2 * 2 * r * d
        mk = lambda: (t16(a_bits), None, t16(b_bits), None)
    # R copies of the weights, so each step reads them from HBM (over the 256 MB Infinity Cache)
    R = max(1, math.ceil(1.0e9 / per_copy)) if T <= 256 else 1
    copies = [mk() for _ in range(R)]
    P = 16 if T <= 256 else 2
    inputs = [(g.tokens(T, 20 + 2 * p), g.tokens(T, 21 + 2 * p)) for p in range(P)]
    dev_in = [(t16(x), t16(yi)) for x, yi in inputs]
    y = torch.empty((T, d), dtype=torch.int16, device=dev)
    ws = tq.alloc_workspace(tq.lib().moe_lowrank_workspace_bytes(T, d, r), dev)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def step(i):
        a, aq, b, bq = copies[i % R]
        x, yi = dev_in[i % P]
        tq.lowrank_apply(x, yi, a, b, r, a_q=aq, b_q=bq, y=y, workspace=ws)

    for i in range(max(warmup, R)):
        step(i)
    torch.cuda.synchronize()
    # events bracket the product A x (stage 0: up to 256 tokens the K-sliced
    # kernel alone, its slices are added up after it) and B z + y_in (stage 1)
    # (on one step in four up to 256 tokens: an event record costs host time
    # that a call of a few microseconds would otherwise pay on every step)
    every = 4 if T <= 256 else 1
    timer = tq.StageTimer((steps + every - 1) // every, stages=[0, 1])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % every == 0:
            with timer.step():
                step(warmup + i)
        else:
            step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    s0, s1 = timer.ms()[0] * 1e-3, timer.ms()[1] * 1e-3
    wbytes = per_copy // 2
    # algorithmic bytes of each product: its weights, its input, its output (and
    # y_in); up to 256 tokens A x leaves fp32 slices, one per K slice
    b0 = wbytes + 2 * T * d + (4 * 8 * T * r if T <= 256 else 2 * T * r)
    b1 = wbytes + 2 * T * r + 2 * 2 * T * d
    flops = 2.0 * T * r * d                 # per product
    # the roofline is the product A x's (the two products take about the same time)
    sec = s0
    kname = "xproj_split_kernel (A x)" if T <= 256 else "split_kernel + dense_gemm_kernel<0> (A x)"
    ms_step = elapsed * 1e3 / steps
    if T <= 256:
        alg = b0
        roof = {"bound": "hbm", "achieved": round(alg / sec / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(alg / sec / 1e9 / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": int(alg)}
    else:
        roof = {"bound": "mfma", "achieved": round(flops / sec / 1e12, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(flops / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                "alg_flops_per_launch": int(flops)}
    roof.update({"traffic": load_traffic(workload, LOWRANK_SOURCES), "kernel": kname,
                 "avg_launch_us": round(sec * 1e6, 2), "timed_steps_with_events": f"1 in {every}"})
    rec = {
        "metric": LOWRANK_METRIC,
        "value": round(steps * T / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"rank-{r} branch y + B(A x) on d={d}, A [{r} x {d}] and B [{d} x {r}] "
                               f"{'as PQ2_0 containers' if ternary else 'in fp16'} "
                               f"({per_copy / 1e6:.2f} MB of weights), {T} token(s) per call",
                   "name": workload, "tokens": T, "weight_replicas": R, "input_sets": P,
                   "parallelism": "single-gpu", "setup_s": round(setup_s, 1)},
        "roofline": roof,
        "stages_us": {"A x": round(s0 * 1e6, 2), "B z + y_in": round(s1 * 1e6, 2)},
        "B_product": {"alg_bytes": int(b1), "achieved_GBs": round(b1 / s1 / 1e9, 1),
                      "hbm_frac": round(b1 / s1 / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if with_cpu:
        step(0)
        torch.cuda.synchronize()
        got = y.cpu().numpy().view(np.uint16)
        print(f"{workload}: timed, {ms_step * 1e3:.1f} us per step; oracle on the host next", file=sys.stderr,
              flush=True)
        rec["cpu_baseline"], rec["parity_max_row_err"] = lowrank_cpu_baseline(*inputs[0], a_bits, b_bits, got)
    del copies, dev_in
    torch.cuda.empty_cache()
    return rec


def calibrate_copy(mib: int, reps: int = 5):
    """Plain device copies of known size: each reads and writes mib MiB once."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=sorted(WORKLOADS) + sorted(QUANT_WORKLOADS) + sorted(PLE_WORKLOADS)
                    + sorted(MTP_WORKLOADS) + sorted(LOWRANK_WORKLOADS))
    ap.add_argument("--sweep", metavar="FILE", help="run every workload, append JSON lines to FILE")
    ap.add_argument("--only", default="", help="comma-separated workloads for --sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="default workload only: skip the extra workloads carried in its record")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run plain device-to-device copies of MIB MiB (the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the block's forward pass is data-parallel over tokens with "
              f"no cross-GPU exchange, so N GPUs run N independent copies of this single-GPU step "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    if not args.no_cpu:
        host_cpu()  # lscpu runs before anything touches the GPU
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.sweep:
        names = [n for n in WORKLOADS if not args.only or n in args.only.split(",")]
        for name in names:
            steps = args.steps if WORKLOADS[name][2] == "decode" else max(5, args.steps // 10)
            rec = run(name, steps, args.warmup, with_cpu=not args.no_cpu)
            with open(args.sweep, "a") as f:
                f.write(json.dumps(rec) + "\n")
            print(f"{name}: {rec['value']:.0f} tokens/s, {rec['ms_per_step']:.4f} ms/step, "
                  f"{rec['roofline']['bound']} frac {rec['roofline']['frac']:.3f}, stages_us "
                  + " ".join(f"{k}={v * 1e3:.1f}" for k, v in rec["stages_ms"].items())
                  + f", parity {rec['parity_max_row_err']:.1e}", file=sys.stderr, flush=True)
        return
    if args.workload in QUANT_WORKLOADS:
        rec = run_quant(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu)
    elif args.workload in PLE_WORKLOADS:
        rec = run_ple(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu)
    elif args.workload in MTP_WORKLOADS:
        rec = run_mtp(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu)
    elif args.workload in LOWRANK_WORKLOADS:
        rec = run_lowrank(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu)
    else:
        rec = run(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu)
        if args.workload == DEFAULT_WORKLOAD and not args.no_extra:
            rec["extra_workloads"] = {}
            for name in EXTRA_WORKLOADS:
                e = run(name, args.steps, args.warmup, with_cpu=False)
                rec["extra_workloads"][name] = {
                    k: e[k] for k in ("value", "unit", "ms_per_step", "roofline", "block", "stages_ms",
                                      "parity_max_row_err")}
                rec["extra_workloads"][name]["workload"] = e["config"]["workload"]
                print(f"{name}: {e['value']:.0f} tokens/s, {e['roofline']['bound']} frac "
                      f"{e['roofline']['frac']:.3f}", file=sys.stderr, flush=True)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Training-step benchmark of the bitwise-reproducible FP32 decoder on one MI355X.

A step is one optimizer step of the whole hot path: for each micro-batch, the
forward pass with cross-entropy and the backward pass folding its gradient into
the accumulator, then AdamW. The default workload is the 162,147,840-parameter
decoder of the MojoLearn 162M model card (12 layers, d 768, 12 heads x 64,
SwiGLU 2048, untied 50,257 tables) with 64 micro-batches of 4 x 2,048 synthetic
Zipf(1.1) token ids per step (524,288 tokens). All token ids of the timed
steps are uploaded to HBM before timing starts.

Prints one JSON line: tokens/s, the step's FP32 TFLOP/s against the MI355X
peak, the roofline of the dominant contraction kernel, and the CPU oracle's
rate on this host's cores on a bounded sample. The first warmup step is traced
in full (HIP events around every dispatch) for the per-kernel table and to name
the dominant kernel; the timed steps bracket only that kernel's call sites with
HIP events, which gives the roofline figure without taxing the throughput with
the tracing of every dispatch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/s + FP32 TFLOP/s %peak at 162M (1 GPU), bit-exact vs oracle"
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def flops_per_token(cfg: dict) -> float:
    """Algorithmic FLOPs per token of one training step: 6 per parameter of the
    matrix products (forward 2, backward 4) plus the causal attention pairs."""
    d, F, L, V, T = cfg["d_model"], cfg["ffn_hidden"], cfg["n_layers"], cfg["vocab"], cfg["seq_len"]
    p_mm = L * (4 * d * d + 3 * d * F) + V * d
    return 6.0 * p_mm + 6.0 * L * d * (T + 1)


# Source files whose change invalidates measured HBM traffic of a kernel family.
_KERNEL_SOURCES = {"k_gemm": "mlb_gemm.hip", "k_tri_nt": "mlb_attn.hip", "k_attn_av": "mlb_attn.hip",
                   "k_attn_rows": "mlb_attn.hip"}


def kernel_source_digest(kernel: str) -> str:
    import hashlib
    csrc = os.path.join(ROOT, "bitwise_reproducible_fp32_amd", "csrc")
    fam = kernel.split("<")[0].strip()
    files = [_KERNEL_SOURCES.get(fam, "mlb_ops.hip"), "mlb_device.hpp"]   # the kernel's code and its device helpers
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, cfg_name: str) -> float | None:
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a
    copy of known size), or None when there is none for this kernel and
    workload or the kernel's source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{cfg_name}.md")
    if not os.path.exists(path):
        return None
    digest = kernel_source_digest(kernel)
    with open(path) as fh:
        for line in fh:
            if not line.startswith("traffic:"):
                continue
            f = dict(kv.split("=", 1) for kv in line[len("traffic:"):].split())
            if f.get("kernel") == kernel.replace(" ", "") and f.get("source_sha256") == digest:
                return float(f["bytes_per_launch"])
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_sample_rate(cfg: dict, cfg_name: str, batch: int, seq_len: int, init: np.ndarray,
                       threads: int) -> dict:
    """One forward+backward of the oracle on a batch x seq_len micro-batch of
    the workload's model (same parameters), timed; the rate is scaled to
    tokens/s of the workload by FLOPs per token."""
    import oracle
    from bitwise_reproducible_fp32_amd import inputs as I
    scfg = dict(cfg, batch=batch, seq_len=seq_len)
    oracle.set_threads(threads)
    m = oracle.Model(scfg, init)
    if cfg_name == "c0":
        x, y = I.c0_batch(0, batch, seq_len)
    else:
        x, y = I.zipf_batch(scfg, 0)
    t0 = time.perf_counter()
    m.forward(x, y)
    m.backward()
    dt = time.perf_counter() - t0
    rate = flops_per_token(scfg) * batch * seq_len / dt
    return {"tokens_per_s": rate / flops_per_token(cfg), "gflops": rate / 1e9, "seconds": dt,
            "threads": threads, "sample": f"{batch}x{seq_len} tokens"}


def cpu_baseline(cfg_name: str, init: np.ndarray) -> dict:
    """The oracle as it stands, on bounded samples of the workload, on this
    host's cores: all of the threads the process may use (OpenMP across
    independent outputs; the OMP_NUM_THREADS share when it is set, else the
    affinity mask), and one thread (the reference semantics). The all-thread
    rate is the reported value."""
    from bitwise_reproducible_fp32_amd import inputs as I
    cfg = I.make_config(cfg_name)
    T = cfg["seq_len"]
    affinity = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or affinity
    many = oracle_sample_rate(cfg, cfg_name, min(2, cfg["batch"]), T, init, threads)
    one = oracle_sample_rate(cfg, cfg_name, 1, min(T, 128), init, 1)
    return {"value": round(many["tokens_per_s"], 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle forward+backward of one {many['sample']} micro-batch of the {cfg_name} model on "
                      f"{threads} threads ({many['seconds']:.1f} s, {many['gflops']:.1f} GFLOP/s), scaled to the "
                      f"workload by FLOPs per token",
            "cpu_model": cpu_model(), "affinity_cpus": affinity,
            "one_thread": {"value": round(one["tokens_per_s"], 2), "unit": "tokens/s",
                           "gflops": round(one["gflops"], 2), "seconds": round(one["seconds"], 1),
                           "sample": f"oracle forward+backward of one {one['sample']} micro-batch on 1 thread"},
            "gflops": round(many["gflops"], 1), "seconds": round(many["seconds"], 1)}


def contraction_kernels(stats: list[dict]) -> dict[str, dict]:
    """Contraction kernel instantiations (records with FLOPs): time, FLOPs, launches and call sites."""
    by_kernel: dict[str, dict] = {}
    for st in stats:
        if st["flops"] > 0:
            k = by_kernel.setdefault(st["kernel"], dict(ms=0.0, flops=0.0, launches=0, sites=set()))
            k["ms"] += st["ms"]; k["flops"] += st["flops"]; k["launches"] += st["launches"]; k["sites"].add(st["site"])
    return by_kernel


def dominant_kernel(stats: list[dict]) -> tuple[str, list[str]]:
    """The contraction instantiation with the most time, and the call sites it ran at."""
    name, k = max(contraction_kernels(stats).items(), key=lambda kv: kv[1]["ms"])
    return name, sorted(k["sites"])


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="c4", choices=["c0", "c3", "c4"])
    ap.add_argument("--micro", type=int, default=0, help="micro-batches per step (default: the config's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--overlap", type=int, default=0, choices=[0, 1],
                    help="run the backward weight-gradient work on the library's second stream (1), or everything "
                         "on one stream (0, default: per-kernel times then measure each kernel alone)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="before the run, negate a MIB-MiB float32 buffer into another (a plain streaming kernel of "
                         "known traffic that scales the HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the step runs on exactly one GPU; the data-parallel path over several "
                                   "GPUs (a fixed-order hand-off of the shard gradients) is not implemented",
                          "n_gpus": a.gpus}))
        return 2

    import torch

    import bitwise_reproducible_fp32_amd as mlb
    from bitwise_reproducible_fp32_amd import inputs as I

    if a.copy_probe > 0:
        n = a.copy_probe * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"# copy probe: {n * 4} bytes read, {n * 4} bytes written", file=sys.stderr, flush=True)
        del src, dst

    cfg = I.make_config(a.config)
    if a.micro:
        cfg["micro"] = a.micro
    S, B, T = cfg["micro"], cfg["batch"], cfg["seq_len"]
    t_setup = time.perf_counter()
    init = I.init_params(cfg)
    torch.cuda.set_device(0)
    model = mlb.Model(cfg, init)
    model.set_overlap(bool(a.overlap))
    nsteps = max(1, a.warmup) + a.steps
    xs = np.empty((nsteps, S, B * T), np.int32)
    ys = np.empty_like(xs)
    for s in range(nsteps):
        for mb in range(S):
            x, y = I.batch_for(a.config, cfg, s + 1, mb)
            xs[s, mb], ys[s, mb] = x.ravel(), y.ravel()
    xd, yd = torch.from_numpy(xs).cuda(), torch.from_numpy(ys).cuda()
    lrs = [I.lr_at(a.config, s + 1) for s in range(nsteps)]
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s; workspace {mlb.workspace_bytes(cfg) / 2**30:.1f} GiB",
          file=sys.stderr, flush=True)

    losses = []

    def step(s: int) -> None:
        for mb in range(S):
            losses.append(float(model.forward_loss(xd[s, mb], yd[s, mb])))
            model.backward()
        model.adamw_step(lrs[s])

    # The first warmup step times every dispatch (HIP events around each, about 5% of step time): it gives the
    # per-kernel table and names the dominant contraction kernel and its call sites. The timed steps then bracket
    # only that kernel's call sites with events, so the throughput is not taxed by the tracing.
    full_stats = None
    for s in range(max(1, a.warmup)):
        if s == 0:
            model.stats_enable(True)
        t0 = time.perf_counter()
        step(s)
        torch.cuda.synchronize()
        if s == 0:
            full_stats = model.stats()
            model.stats_enable(False)
        print(f"# warmup step {s + 1}: {time.perf_counter() - t0:.2f}s", file=sys.stderr, flush=True)
    dom_name, dom_sites = dominant_kernel(full_stats)
    model.stats_sites(dom_sites)
    model.stats_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(max(1, a.warmup), max(1, a.warmup) + a.steps):
        ts = time.perf_counter()
        step(s)
        print(f"# step {s + 1}: {time.perf_counter() - ts:.2f}s loss {losses[-1]:.5f}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed_stats = model.stats()
    model.stats_enable(False)
    model.stats_sites(None)

    # inference surface (not part of the training metric): forward with loss
    # and kept logits, and greedy next-token choices, on the same batches
    inf_iters = 5
    torch.cuda.synchronize()
    t_inf = time.perf_counter()
    for i in range(inf_iters):
        model.infer(xd[0, i % S], yd[0, i % S])
    t_inf = (time.perf_counter() - t_inf) / inf_iters
    t_gr = time.perf_counter()
    for i in range(inf_iters):
        model.greedy_next(xd[0, i % S], T - 1)
    t_gr = (time.perf_counter() - t_gr) / inf_iters
    print("# per-kernel table of the first (untimed, fully traced) step:", file=sys.stderr)
    for st in sorted(full_stats, key=lambda t: -t["ms"]):
        rate = (f"{st['flops'] / st['ms'] / 1e9:7.2f} TFLOP/s" if st["flops"] else
                f"{st['bytes'] / st['ms'] / 1e6:7.1f} GB/s")
        print(f"# {st['ms']:9.2f} ms/step {st['launches']:5d}x {rate}  {st['site']:14s} "
              f"{st['kernel']}", file=sys.stderr)

    tokens = S * B * T
    fpt = flops_per_token(cfg)
    value = tokens * a.steps / elapsed
    tflops = fpt * tokens * a.steps / elapsed / 1e12

    # the dominant kernel's dispatches inside the timed region (only its call sites were traced there)
    dom = dict(ms=0.0, flops=0.0, launches=0)
    for st in timed_stats:
        if st["kernel"] == dom_name:
            dom["ms"] += st["ms"]; dom["flops"] += st["flops"]; dom["launches"] += st["launches"]
    dom_avg_ms = dom["ms"] / dom["launches"]
    dom_achieved = dom["flops"] / dom["launches"] / (dom_avg_ms / 1e3) / 1e12
    by_kernel = contraction_kernels(full_stats)
    gemm_ms = sum(k["ms"] for k in by_kernel.values())
    gemm_flops = sum(k["flops"] for k in by_kernel.values())
    total_ms = sum(st["ms"] for st in full_stats)
    mem_sites = {}
    for st in full_stats:
        if st["bytes"] > 0:
            key = st["site"] if st["kernel"] == st["site"] else f'{st["site"]}:{st["kernel"]}'
            r = mem_sites.setdefault(key, dict(ms=0.0, bytes=0.0, launches=0))
            r["ms"] += st["ms"]; r["bytes"] += st["bytes"]; r["launches"] += st["launches"]

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(elapsed / a.steps * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": ("synthetic (seeded order-2 Markov bytes, N(0,0.02) init)" if a.config == "c0" else
                 "synthetic (seeded Zipf(1.1) token ids, N(0,0.02) init)"),
        "config": {"workload": f"{a.config}: {I.param_count(cfg):,}-param decoder, {S} micro-batches of "
                               f"{B}x{T} tokens per step", "tokens_per_step": tokens, "micro_batches": S,
                   "batch": B, "seq_len": T, "parallelism": "none (1 GPU)", "stream_overlap": bool(a.overlap)},
        "tflops": round(tflops, 2),
        "pct_fp32_peak": round(100 * tflops / PEAK_FP32_TFLOPS, 2),
        "flops_per_token": fpt,
        "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": round(dom_achieved, 2),
                     "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s", "frac": round(dom_achieved / PEAK_FP32_TFLOPS, 4),
                     "traffic": measured_traffic(dom_name, a.config), "avg_ms": round(dom_avg_ms, 4), "launches": dom["launches"],
                     "flops_per_launch": dom["flops"] / dom["launches"], "sites": sorted(dom_sites),
                     "timing": "HIP events around the dominant kernel's call sites in the timed steps"},
        "contractions": {"ms_share": round(gemm_ms / total_ms, 4) if total_ms else None,
                         "tflops": round(gemm_flops / (gemm_ms / 1e3) / 1e12, 2) if gemm_ms else None,
                         "from": "first (untimed, fully traced) step"},
        "hbm_kernels": {k: {"GB/s": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1), "ms": round(v["ms"], 3)}
                        for k, v in sorted(mem_sites.items(), key=lambda kv: -kv[1]["ms"])[:8]},
        "loss_first_last": [losses[0], losses[-1]],
        "inference": {"tokens_per_s": round(B * T / t_inf, 1), "ms_per_batch": round(t_inf * 1e3, 2),
                      "greedy_next_ms": round(t_gr * 1e3, 2),
                      "what": f"forward + loss of one {B}x{T} batch with logits kept; greedy next token of {B} "
                              f"sequences at position {T - 1} (a full forward each)"},
    }
    if not a.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(a.config, init)
        except Exception as e:  # the baseline is reported, never required
            out["cpu_baseline"] = {"error": str(e)}
    print(json.dumps(out), flush=True)
    model.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())

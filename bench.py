"""Benchmark of the paged-KV attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the path over the Llama-3-8B-shaped decode batch
(B=64, contexts U[128,4096], h_q=32, h_kv=8, d_h=128, bf16, 16-token blocks,
pool = used blocks + 10% free, shuffled): kv_append of the 64 new tokens, then
paged_decode_attention over every context.  Inputs are seeded synthetic data
already resident in HBM; three copies of the pool are rotated so that no step
finds its KV data in the 256 MB Infinity Cache or the L2s left by the step
before.  K steps are timed with wall clock between two synchronisations.

Printed as one JSON line:
  value      KV bytes attended per second (GB/s), whole step (append + decode)
  roofline   the decode call (its kernels timed by HIP events on the launch
             stream) against the 8 TB/s HBM peak, algorithmic bytes per launch
             = sum_b L_b * 2 * h_kv * d_h * 2 B (KV-cache footprint per token of
             one layer, LLM Inference Server page, Required Mathematical
             Concepts)
  prefill    paged_prefill_attention on the mixed Qwen2.5-0.5B-shaped batch
             (4 prompts x 512 tokens, h_q=14, h_kv=2, d_h=64) in TFLOP/s
  cpu_baseline  the CPU oracle on the same decode step, on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

from paged_kv_cache_274_amd import ops
from paged_kv_cache_274_amd import workloads as W

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attention: KV GB/s read and % of HBM peak; prefill TFLOP/s"


def kv_bytes(w: W.Workload) -> int:
    """Algorithmic KV bytes one decode call reads: 2 * h_kv * d_h * elem per context token."""
    return int(w.dec_context_lens.to(torch.int64).sum()) * 2 * w.h_kv * w.d * w.elem_bytes


def prefill_flops(w: W.Workload) -> int:
    """2 * d_h flops for QK^T and 2 * d_h for PV per (query head, visible key) pair."""
    total_pairs = 0
    for s in range(w.S):
        L = int(w.pre_context_lens[s])
        n = int(w.pre_cu_seqlens[s + 1] - w.pre_cu_seqlens[s])
        total_pairs += sum(L - n + i + 1 for i in range(n))
    return 4 * w.d * w.h_q * total_pairs


class Resident:
    """Device copies of one workload; the pool is replicated `copies` times."""

    def __init__(self, w: W.Workload, dev: str, copies: int = 1):
        self.w = w
        self.q = w.dec_q.to(dev)
        self.k_new = w.k_new.to(dev)
        self.v_new = w.v_new.to(dev)
        self.slots = w.slot_mapping.to(dev)
        self.tables = w.dec_block_tables.to(dev)
        self.lens = w.dec_context_lens.to(dev)
        self.pre_q = w.pre_q.to(dev)
        self.cu = w.pre_cu_seqlens.to(dev)
        self.pre_tables = w.pre_block_tables.to(dev)
        self.pre_lens = w.pre_context_lens.to(dev)
        self.pools = [(w.k_cache.to(dev), w.v_cache.to(dev)) for _ in range(copies)]
        self.out = torch.empty_like(self.q)
        self.pre_out = torch.empty_like(self.pre_q)
        nbytes = ops.decode_workspace_bytes(w.B, w.h_q, w.h_kv, w.d, w.dec_max_context_len, w.dtype)
        self.ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)

    def append(self, i: int):
        kc, vc = self.pools[i % len(self.pools)]
        ops.kv_append(self.k_new, self.v_new, self.slots, kc, vc)

    def decode(self, i: int):
        kc, vc = self.pools[i % len(self.pools)]
        ops.paged_decode_attention(self.q, kc, vc, self.tables, self.lens,
                                   self.w.dec_max_context_len, scale=self.w.scale,
                                   out=self.out, workspace=self.ws)

    def prefill(self, i: int):
        kc, vc = self.pools[i % len(self.pools)]
        ops.paged_prefill_attention(self.pre_q, self.cu, kc, vc, self.pre_tables, self.pre_lens,
                                    self.w.pre_max_q_len, scale=self.w.scale, out=self.pre_out)


def time_decode_step(r: Resident, steps: int, warmup: int):
    for i in range(warmup):
        r.append(i)
        r.decode(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        r.append(i)
        ev[i][0].record()
        r.decode(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = [a.elapsed_time(b) for a, b in ev]
    return wall, dec_ms


def time_prefill(r: Resident, iters: int = 50, warmup: int = 5):
    for i in range(warmup):
        r.prefill(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        r.prefill(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def cpu_baseline(w: W.Workload, reps: int):
    """The oracle (append + decode of the whole step) on the host cores."""
    import oracle.attention as O
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    q = w.dec_q.to(torch.float64).numpy()
    kc = w.k_cache.to(torch.float64).numpy()
    vc = w.v_cache.to(torch.float64).numpy()
    kn = w.k_new.to(torch.float64).numpy()
    vn = w.v_new.to(torch.float64).numpy()
    times = []
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        for _ in range(reps):
            t0 = time.perf_counter()
            k2, v2 = O.kv_append(kn, vn, w.slot_mapping.numpy(), kc, vc)
            O.decode(q, k2, v2, w.dec_block_tables.numpy(), w.dec_context_lens.numpy(), w.scale)
            times.append(time.perf_counter() - t0)
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    med = statistics.median(times)
    return {"value": round(kv_bytes(w) / med / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"whole decode step of the same workload (kv_append + decode, "
                      f"{w.B} sequences, {int(w.dec_context_lens.sum())} context tokens), "
                      f"median of {reps} runs, float64 NumPy with BLAS pinned to 1 thread, "
                      f"{sum(times):.1f} s total; host {os.cpu_count()} CPUs"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--cpu-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(the per-GPU workload is already one GPU's share); run with --gpus 1",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = "cuda:0"
    ops.lib()

    w3 = W.config(3)
    r3 = Resident(w3, dev, copies=args.copies)
    wall, dec_ms = time_decode_step(r3, args.steps, args.warmup)
    kvb = kv_bytes(w3)
    value = kvb * args.steps / wall / 1e9
    dec_avg_s = statistics.mean(dec_ms) / 1e3
    achieved = kvb / dec_avg_s / 1e9
    del r3
    torch.cuda.empty_cache()

    w5 = W.config(5)
    r5 = Resident(w5, dev)
    r5.append(0)
    pf_ms = time_prefill(r5)
    pf_avg_s = statistics.mean(pf_ms) / 1e3
    pf_tflops = prefill_flops(w5) / pf_avg_s / 1e12
    del r5
    torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)",
        "config": {
            "workload": "llama3-8b-shaped decode step: B=64, contexts U[128,4096], h_q=32, "
                        "h_kv=8, d_h=128, bf16, 16-token blocks, shuffled pool +10% free",
            "context_tokens": int(w3.dec_context_lens.sum()),
            "kv_bytes_per_step": kvb,
            "n_blocks": w3.n_blocks,
            "num_splits": ops.decode_num_splits(w3.B, w3.h_q, w3.h_kv, w3.d,
                                                w3.dec_max_context_len, w3.dtype),
            "pool_copies_rotated": args.copies,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_decode_attention (split pass + combine pass)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_us": round(dec_avg_s * 1e6, 2),
        },
        "prefill": {
            "workload": "qwen2.5-0.5b-shaped prefill: 4 prompts x 512 tokens, h_q=14, h_kv=2, "
                        "d_h=64, causal, bf16",
            "flops": prefill_flops(w5),
            "avg_us": round(pf_avg_s * 1e6, 2),
            "tflops": round(pf_tflops, 3),
            "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
            "frac": round(pf_tflops / BF16_MFMA_PEAK_TFLOPS, 5),
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w3, args.cpu_reps)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

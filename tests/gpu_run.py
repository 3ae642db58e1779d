"""Run a seeded workload through the HIP path (C-ABI via the ctypes binding)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from paged_kv_cache_274_amd import ops
from paged_kv_cache_274_amd import workloads as W

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


@dataclass
class GpuResult:
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    decode: Optional[torch.Tensor]
    prefill: Optional[torch.Tensor]


def run(w: W.Workload, dev="cuda:0", num_splits=0, append=True, do_decode=True,
        do_prefill=True) -> GpuResult:
    kc = w.k_cache.to(dev)
    vc = w.v_cache.to(dev)
    if append and w.T:
        ops.kv_append(w.k_new.to(dev), w.v_new.to(dev), w.slot_mapping.to(dev), kc, vc)
    dec = pre = None
    if do_prefill and w.S:
        pre = ops.paged_prefill_attention(
            w.pre_q.to(dev), w.pre_cu_seqlens.to(dev), kc, vc, w.pre_block_tables.to(dev),
            w.pre_context_lens.to(dev), w.pre_max_q_len, scale=w.scale)
    if do_decode and w.B:
        dec = ops.paged_decode_attention(
            w.dec_q.to(dev), kc, vc, w.dec_block_tables.to(dev), w.dec_context_lens.to(dev),
            w.dec_max_context_len, scale=w.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return GpuResult(kc.cpu(), vc.cpu(), None if dec is None else dec.cpu(),
                     None if pre is None else pre.cpu())


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def max_err(got: torch.Tensor, ref: np.ndarray) -> float:
    g = got.to(torch.float64).numpy()
    assert not np.isnan(g).any(), "NaN in GPU output"
    return float(np.max(np.abs(g - ref))) if g.size else 0.0

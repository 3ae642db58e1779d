"""paged_decode_attention_noalloc (the decode entry point that allocates
nothing: its workspace is the library's static device array) against
paged_decode_attention on the same inputs, through the C ABI.

Two calls in a row, the second on a smaller batch: the Llama-3-8B-shaped decode
batch (64 sequences, contexts U[128,4096], 32/8/128, bf16), then the
Llama-3.2-1B-shaped one (8 x 512, 32/8/64).  The two entry points run the same
kernels with the same automatic split, so the outputs must agree bit for bit,
and both must be within the bf16 bound (2e-2) of the oracle.  The device's
free memory must not change across the calls.
"""
import numpy as np
import pytest
import torch

import oracle.attention as O
from gpu_run import bits, max_err
from paged_kv_cache_274_amd import ops
from paged_kv_cache_274_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(k):
    w = W.config(k, poison=True)
    kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
    ops.kv_append(w.k_new.to(DEV), w.v_new.to(DEV), w.slot_mapping.to(DEV), kc, vc)
    return w, kc, vc, w.dec_q.to(DEV), w.dec_block_tables.to(DEV), w.dec_context_lens.to(DEV)


def _oracle(w):
    f64 = lambda t: t.to(torch.float64).numpy()  # noqa: E731
    k_ref, v_ref = O.kv_append(f64(w.k_new), f64(w.v_new), w.slot_mapping.numpy(),
                               f64(w.k_cache), f64(w.v_cache))
    return O.decode(f64(w.dec_q), k_ref, v_ref, w.dec_block_tables.numpy(),
                    w.dec_context_lens.numpy(), w.scale)


def test_noalloc_matches_the_allocating_entry_point_twice():
    ops.lib()
    cases = []
    for k in (3, 2):        # the second call is on a smaller batch
        print(f"noalloc: preparing config {k}", flush=True)
        cases.append(_inputs(k))
    torch.cuda.synchronize()
    free0 = None
    for w, kc, vc, q, tbl, lens in cases:
        print(f"noalloc: B={w.B} h_q={w.h_q} h_kv={w.h_kv} d={w.d}", flush=True)
        out_s = torch.empty_like(q)
        ops.paged_decode_attention_noalloc(q, kc, vc, tbl, lens, w.dec_max_context_len, out_s,
                                           scale=w.scale)
        torch.cuda.synchronize()
        if free0 is None:
            free0 = torch.cuda.mem_get_info()[0]
        out_a = ops.paged_decode_attention(q, kc, vc, tbl, lens, w.dec_max_context_len,
                                           scale=w.scale)
        out_s2 = torch.empty_like(q)
        free1 = torch.cuda.mem_get_info()[0]
        ops.paged_decode_attention_noalloc(q, kc, vc, tbl, lens, w.dec_max_context_len, out_s2,
                                           scale=w.scale)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free1, "the no-alloc call changed free memory"
        a, s, s2 = out_a.cpu(), out_s.cpu(), out_s2.cpu()
        assert torch.equal(bits(s), bits(a)) and torch.equal(bits(s2), bits(a))
        err = max_err(s, _oracle(w))
        print(f"noalloc: max|err| vs oracle {err:.3e}", flush=True)
        assert err <= 2e-2

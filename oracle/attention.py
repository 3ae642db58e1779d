"""CPU oracle for attention over a block-paged KV cache (float64, NumPy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library (``paged_kv_cache_274_amd``) never does, and this module imports
nothing from it: the two share no code.  Inputs come from the seeded
generators as plain arrays.

What it computes is the plain definition of the operations, written out:

* ``kv_append``: copy each new token's K and V rows (all KV heads) into the pool
  slot its slot number names, in place, with no reallocation.  This is the
  pre-allocated cache that is written in place at the current length instead
  of being concatenated ("KV-Cache Engine" stage of the LLM Inference Server
  page, pre-allocation task, and its LayerKVCache reference class, which writes
  the new rows at the current length and then returns the cache up to the new
  length).  Pool slots are fixed 16-token physical blocks reached through a
  per-sequence block table (same page, "Paged KV-Cache Block Allocator"
  stretch challenge; "block table / paged KV slots" box of the pipeline figure
  on the "LLM Inference Server From Scratch" page).

* ``decode``: for every sequence b and query head h, softmax of the scaled dot
  products of q[b, h] with the keys of all L_b context tokens (the appended one
  included), times their values.  This is single-token decode attending over
  the whole cached context (LLM Inference Server page, Stage 1 prefill/decode
  task: each decode step feeds only the new token, at start_pos = current
  length).

* ``prefill``: for sequence s with n_s new query tokens at positions
  L_s - n_s .. L_s - 1, the query at position p attends to keys 0..p inclusive
  (causal masking named in the "Attention Kernel" box of the pipeline figure
  and in "What you build" on the From Scratch page; the prompt is processed in
  parallel, LLM Inference Server page, Stage 1 prefill/decode task).

Grouped-query attention ("GQA" in the same figure box): query head h reads KV
head ``h // (h_q // h_kv)``.  The scale is passed in (the pages' tool,
PyTorch's scaled_dot_product_attention, defaults to 1/sqrt(d_h)).

Numbers: every input is widened to float64 before any arithmetic, so bf16
inputs are used at their exact stored values; the result stays float64.  A
context of length 0 yields zeros.

Each readable step is a small named helper (``kv_head_of``, ``slot_to_block``,
``key_limit``, ``gather_sequence``, ``dot_scores``, ``softmax_weighted_sum``) so that a test can
plant a mistake in exactly one of them and check that the pins catch it.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, h_q: int, h_kv: int) -> int:
    """KV head read by query head h: consecutive groups of h_q / h_kv query heads."""
    return h // (h_q // h_kv)


def slot_to_block(slot: int):
    """Physical (block, offset) of a slot number, slot = block * 16 + offset."""
    return slot // BLOCK, slot % BLOCK


def key_limit(L: int, n: int, i: int) -> int:
    """Number of keys visible to query i of a sequence with context L and n queries.

    Query i sits at absolute position p = L - n + i and sees keys 0..p inclusive.
    """
    return L - n + i + 1


def dot_scores(keys: np.ndarray, queries: np.ndarray, scale: float) -> np.ndarray:
    """scale * <query_i, key_j> for queries [n, d] and keys [L, d]; result [n, L]."""
    return scale * (queries @ keys.T)


def gather_sequence(cache: np.ndarray, table_row, L: int) -> np.ndarray:
    """Logical [L, h_kv, d] view of one sequence: token t lives in
    block table_row[t // 16] at offset t % 16."""
    h_kv, d = cache.shape[1], cache.shape[3]
    out = np.empty((L, h_kv, d), dtype=np.float64)
    for t in range(L):
        out[t] = cache[int(table_row[t // BLOCK]), :, t % BLOCK, :]
    return out


def softmax_weighted_sum(scores: np.ndarray, values: np.ndarray) -> np.ndarray:
    """sum_j softmax(scores)_j * values[j]; scores [L], values [L, d]."""
    if scores.shape[0] == 0:
        return np.zeros(values.shape[1], dtype=np.float64)
    w = np.exp(scores - scores.max())
    return (w @ values) / w.sum()


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache):
    """Return copies of the pools with the new rows written at their slots.

    A negative slot means "no write" (padding).  Duplicate non-negative slots
    and slots outside the pool are caller errors and raise ValueError.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    slots = [int(s) for s in np.asarray(slot_mapping).reshape(-1)]
    n_slots = k_out.shape[0] * BLOCK
    live = [s for s in slots if s >= 0]
    if len(set(live)) != len(live):
        raise ValueError("duplicate slot in slot_mapping")
    if any(s >= n_slots for s in live):
        raise ValueError("slot outside the pool")
    for i, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = slot_to_block(s)
        k_out[blk, :, off, :] = k_new[i]
        v_out[blk, :, off, :] = v_new[i]
    return k_out, v_out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float) -> np.ndarray:
    """out[b, h] = softmax_j(scale * <q[b,h], K_b[j, g(h)]>) . V_b[:, g(h)], j < L_b."""
    q = _f64(q)
    k_cache = _f64(k_cache)
    v_cache = _f64(v_cache)
    B, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    out = np.zeros((B, h_q, d), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        K = gather_sequence(k_cache, block_tables[b], L)
        V = gather_sequence(v_cache, block_tables[b], L)
        for h in range(h_q):
            g = kv_head_of(h, h_q, h_kv)
            s = dot_scores(K[:, g, :], q[b, h][None, :], scale)[0]
            out[b, h] = softmax_weighted_sum(s, V[:, g, :])
    return out


def prefill(q, cu_seqlens, k_cache, v_cache, block_tables, context_lens, scale: float) -> np.ndarray:
    """Causal attention of packed query rows over each sequence's paged context.

    Rows cu_seqlens[s] .. cu_seqlens[s+1]-1 are the n_s queries of sequence s;
    query i of it sees keys 0 .. key_limit(L_s, n_s, i) - 1.
    """
    q = _f64(q)
    k_cache = _f64(k_cache)
    v_cache = _f64(v_cache)
    T_q, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    out = np.zeros((T_q, h_q, d), dtype=np.float64)
    S = len(context_lens)
    for s in range(S):
        lo, hi = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        n = hi - lo
        L = int(context_lens[s])
        if n > L:
            raise ValueError("more queries than context")
        K = gather_sequence(k_cache, block_tables[s], L)
        V = gather_sequence(v_cache, block_tables[s], L)
        for h in range(h_q):
            g = kv_head_of(h, h_q, h_kv)
            scores = dot_scores(K[:, g, :], q[lo:hi, h, :], scale)      # [n, L]
            for i in range(n):
                lim = key_limit(L, n, i)
                out[lo + i, h] = softmax_weighted_sum(scores[i, :lim], V[:lim, g, :])
    return out

"""Seeded synthetic inputs for paged-KV attention.

This module only *constructs inputs*: context lengths, the assignment of physical
16-token blocks to sequences (block tables), the write slots of the new tokens
(slot mapping) and the N(0,1) value draws.  It holds none of the attention
arithmetic, so the CPU oracle and the HIP path can both be fed from it without
sharing any computation.

The shapes follow the workloads the pages describe: a block pool of fixed
16-token blocks behind a per-sequence block table ("Paged KV-Cache Block
Allocator", LLM Inference Server page, Optional Stretch Challenges), single-token
decode for a continuous batch of variable-length sequences and causal prefill of
new prompts (Stage 1, prefill/decode task), and a shared system-prompt prefix
(Stage 1, prefix-cache task).

Conventions (all are input layout, not arithmetic):

* K/V pools are ``[n_blocks, h_kv, 16, d]``.
* A sequence with context length ``L`` (counting the tokens appended this step)
  and ``n`` new tokens holds ``L - n`` prior tokens in the pool; the ``n`` new
  tokens go to positions ``L - n .. L - 1``.
* ``slot = physical_block * 16 + offset``; the new token at position ``p`` of a
  sequence with table ``tbl`` has slot ``tbl[p // 16] * 16 + p % 16``.
* Draw order with ``rng``: context lengths (by the caller), block permutation,
  q (decode rows, then prefill rows), k_new, v_new, pool K, pool V.
* Values are float32 N(0,1), cast to the storage dtype by torch (round to
  nearest even for bfloat16).
* With ``poison=True`` every pool slot that does not hold a prior token (free
  blocks, tails of last blocks, the slots the append will fill) is NaN, so an
  unmasked read shows up as NaN in the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

BLOCK = 16

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    h_q: int
    h_kv: int
    d: int
    scale: float                 # a float32-representable value
    n_blocks: int
    max_blocks_per_seq: int
    k_cache: torch.Tensor        # [n_blocks, h_kv, 16, d], before the append
    v_cache: torch.Tensor
    k_new: torch.Tensor          # [T, h_kv, d]  (prefill tokens first, then decode tokens)
    v_new: torch.Tensor
    slot_mapping: torch.Tensor   # int64 [T]
    dec_q: torch.Tensor          # [B, h_q, d]
    dec_block_tables: torch.Tensor   # int32 [B, max_blocks_per_seq]
    dec_context_lens: torch.Tensor   # int32 [B]
    pre_q: torch.Tensor          # [T_q, h_q, d] packed rows of all prefill sequences
    pre_cu_seqlens: torch.Tensor     # int32 [S + 1]
    pre_block_tables: torch.Tensor   # int32 [S, max_blocks_per_seq]
    pre_context_lens: torch.Tensor   # int32 [S]
    shared_prefix_blocks: int = 0

    @property
    def B(self) -> int:
        return int(self.dec_q.shape[0])

    @property
    def S(self) -> int:
        return int(self.pre_context_lens.shape[0])

    @property
    def T(self) -> int:
        return int(self.k_new.shape[0])

    @property
    def T_q(self) -> int:
        return int(self.pre_q.shape[0])

    @property
    def dec_max_context_len(self) -> int:
        return int(self.dec_context_lens.max()) if self.B else 0

    @property
    def pre_max_q_len(self) -> int:
        if self.S == 0:
            return 0
        cu = self.pre_cu_seqlens
        return int((cu[1:] - cu[:-1]).max())

    @property
    def elem_bytes(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()


def _draw(rng: np.random.Generator, shape: Tuple[int, ...]) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def _cast(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(a).to(dtype)


def build(
    name: str,
    rng: np.random.Generator,
    *,
    dtype: str,
    h_q: int,
    h_kv: int,
    d: int,
    decode_lens: Sequence[int] = (),
    prefill: Sequence[Tuple[int, int]] = (),
    pool_blocks: Optional[int] = None,
    free_frac: float = 0.0,
    shared_prefix_blocks: int = 0,
    max_blocks_per_seq: Optional[int] = None,
    scale: Optional[float] = None,
    poison: bool = False,
) -> Workload:
    """Build one workload.

    ``decode_lens``: context length of each decode sequence (one new token each).
    ``prefill``: ``(context_len, n_new)`` for each prefill sequence.
    ``pool_blocks``: explicit pool size; otherwise ``N + ceil(free_frac * N)`` with
    ``N`` the number of distinct blocks the sequences use.
    ``shared_prefix_blocks``: that many leading logical blocks of every *decode*
    sequence map to the same physical blocks (a shared system prompt).
    """
    tdtype = _DTYPES[dtype]
    seqs: List[Tuple[int, int, bool]] = [(int(L), int(n), False) for L, n in prefill]
    seqs += [(int(L), 1, True) for L in decode_lens]
    for L, n, _ in seqs:
        if not (0 <= n <= L):
            raise ValueError(f"bad sequence (L={L}, n={n})")
    P = int(shared_prefix_blocks)
    for L, n, is_dec in seqs:
        if is_dec and P and P * BLOCK > L - n:
            raise ValueError("shared prefix must hold prior tokens only")

    nblk = [-(-L // BLOCK) for L, _, _ in seqs]
    used = P + sum(nb - (P if is_dec else 0) for nb, (_, _, is_dec) in zip(nblk, seqs))
    n_blocks = pool_blocks if pool_blocks is not None else used + math.ceil(free_frac * used)
    if n_blocks < used:
        raise ValueError(f"pool of {n_blocks} blocks cannot hold {used} used blocks")
    mb = max_blocks_per_seq if max_blocks_per_seq is not None else max(nblk + [1])
    if mb < max(nblk + [0]):
        raise ValueError("max_blocks_per_seq too small")

    # 2. physical block permutation; ids are handed out in order.
    perm = rng.permutation(n_blocks).astype(np.int64)
    shared = perm[:P]
    ptr = P
    tables = []
    for nb, (L, n, is_dec) in zip(nblk, seqs):
        own = nb - (P if is_dec else 0)
        row = list(shared) if (is_dec and P) else []
        row += list(perm[ptr:ptr + own])
        ptr += own
        tables.append(row)
    free_ids = perm[ptr:]
    filler = int(free_ids[0]) if len(free_ids) else 0

    # 3. q (decode rows, then prefill rows); 4. new K/V; 5. pool K then V.
    B = sum(1 for s in seqs if s[2])
    T_q = sum(n for L, n, is_dec in seqs if not is_dec)
    T = sum(n for _, n, _ in seqs)
    dec_q = _draw(rng, (B, h_q, d))
    pre_q = _draw(rng, (T_q, h_q, d))
    k_new = _draw(rng, (T, h_kv, d))
    v_new = _draw(rng, (T, h_kv, d))
    k_pool = _draw(rng, (n_blocks, h_kv, BLOCK, d))
    v_pool = _draw(rng, (n_blocks, h_kv, BLOCK, d))

    slots = []
    for row, (L, n, _) in zip(tables, seqs):
        for p in range(L - n, L):
            slots.append(int(row[p // BLOCK]) * BLOCK + p % BLOCK)

    if poison:
        holds_prior = np.zeros((n_blocks, BLOCK), dtype=bool)
        for row, (L, n, _) in zip(tables, seqs):
            for p in range(L - n):
                holds_prior[row[p // BLOCK], p % BLOCK] = True
        dead = ~holds_prior
        k_pool.transpose(0, 2, 1, 3)[dead] = np.nan
        v_pool.transpose(0, 2, 1, 3)[dead] = np.nan

    def table_tensor(rows):
        t = np.full((len(rows), mb), filler, dtype=np.int32)
        for i, r in enumerate(rows):
            t[i, :len(r)] = r
        return torch.from_numpy(t)

    pre_rows = [t for t, s in zip(tables, seqs) if not s[2]]
    dec_rows = [t for t, s in zip(tables, seqs) if s[2]]
    pre_n = [n for L, n, is_dec in seqs if not is_dec]
    cu = np.zeros(len(pre_n) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(pre_n, dtype=np.int64)

    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scale = float(np.float32(scale))

    return Workload(
        name=name, dtype=tdtype, h_q=h_q, h_kv=h_kv, d=d, scale=scale,
        n_blocks=n_blocks, max_blocks_per_seq=mb,
        k_cache=_cast(k_pool, tdtype), v_cache=_cast(v_pool, tdtype),
        k_new=_cast(k_new, tdtype), v_new=_cast(v_new, tdtype),
        slot_mapping=torch.tensor(slots, dtype=torch.int64),
        dec_q=_cast(dec_q, tdtype),
        dec_block_tables=table_tensor(dec_rows),
        dec_context_lens=torch.tensor([L for L, _, d_ in seqs if d_], dtype=torch.int32),
        pre_q=_cast(pre_q, tdtype),
        pre_cu_seqlens=torch.from_numpy(cu),
        pre_block_tables=table_tensor(pre_rows),
        pre_context_lens=torch.tensor([L for L, _, d_ in seqs if not d_], dtype=torch.int32),
        shared_prefix_blocks=P,
    )


CONFIG_NAMES = {
    1: "tiny-decode-fp32 (B=2, L=17/40, h_q=4, h_kv=2, d=64)",
    2: "llama3.2-1b-decode-bf16 (B=8, L=512, h_q=32, h_kv=8, d=64)",
    3: "llama3-8b-decode-bf16 (B=64, L~U[128,4096], h_q=32, h_kv=8, d=128)",
    4: "long-context-prefix-shared-decode-bf16 (B=8, L=8192, 13 shared blocks, h_q=32, h_kv=8, d=128)",
    5: "qwen2.5-0.5b-mixed-bf16 (prefill 4x512 + 60 decode L~U[64,2048], h_q=14, h_kv=2, d=64)",
}


def config(k: int, *, poison: bool = False) -> Workload:
    """The five seeded workloads, ``rng = default_rng(274000 + k)``."""
    rng = np.random.default_rng(274000 + k)
    name = CONFIG_NAMES[k]
    if k == 1:
        return build(name, rng, dtype="f32", h_q=4, h_kv=2, d=64, decode_lens=[17, 40],
                     pool_blocks=16, scale=0.125, poison=poison)
    if k == 2:
        return build(name, rng, dtype="bf16", h_q=32, h_kv=8, d=64, decode_lens=[512] * 8,
                     poison=poison)
    if k == 3:
        lens = rng.integers(128, 4096, size=64, endpoint=True)
        return build(name, rng, dtype="bf16", h_q=32, h_kv=8, d=128, decode_lens=lens,
                     free_frac=0.10, poison=poison)
    if k == 4:
        return build(name, rng, dtype="bf16", h_q=32, h_kv=8, d=128, decode_lens=[8192] * 8,
                     shared_prefix_blocks=13, poison=poison)
    if k == 5:
        lens = rng.integers(64, 2048, size=60, endpoint=True)
        return build(name, rng, dtype="bf16", h_q=14, h_kv=2, d=64, decode_lens=lens,
                     prefill=[(512, 512)] * 4, free_frac=0.10, poison=poison)
    raise ValueError(f"no config {k}")


@dataclass
class Int8Pools:
    """An INT8 cache beside a workload: codes int8 ``[n_blocks, h_kv, 16, d]`` and
    float32 scales ``[n_blocks, h_kv, 16]`` for K and for V."""
    k_codes: torch.Tensor
    v_codes: torch.Tensor
    k_scales: torch.Tensor
    v_scales: torch.Tensor


def int8_pools(w: Workload, seed: int, poison: bool = False) -> Int8Pools:
    """Random INT8 pools of the workload's shape: codes uniform on [-127, 127] and
    scales uniform on [0.005, 0.03] (the scale range that rows of N(0,1) values
    get), drawn with ``default_rng(seed)`` in the order K codes, V codes, K
    scales, V scales.  These are draws, not the quantisation of anything.  With
    ``poison=True`` the scales of every slot the workload's bf16 pool marks
    unused (NaN there) are NaN, so an unmasked read shows up as NaN."""
    rng = np.random.default_rng(seed)
    shape = tuple(w.k_cache.shape)
    kq = rng.integers(-127, 128, size=shape).astype(np.int8)
    vq = rng.integers(-127, 128, size=shape).astype(np.int8)
    ks = rng.uniform(0.005, 0.03, size=shape[:3]).astype(np.float32)
    vs = rng.uniform(0.005, 0.03, size=shape[:3]).astype(np.float32)
    if poison:
        unused = torch.isnan(w.k_cache[..., 0].float()).numpy()
        ks[unused] = np.nan
        vs[unused] = np.nan
    return Int8Pools(torch.from_numpy(kq), torch.from_numpy(vq), torch.from_numpy(ks),
                     torch.from_numpy(vs))


def long_prefill(h_q: int, h_kv: int, d: int, prompts: int = 4, length: int = 4096,
                 seed: int = 274020) -> Workload:
    """Long causal prompts prefilled whole (``prompts`` x ``length`` tokens, the
    K/V of every token already appended), for measuring the prefill kernel away
    from its launch ramp.  Pool = used blocks + 10% free, shuffled."""
    return build(f"prefill-{prompts}x{length}-{h_q}/{h_kv}/{d}", np.random.default_rng(seed),
                 dtype="bf16", h_q=h_q, h_kv=h_kv, d=d,
                 prefill=[(length, length)] * prompts, free_frac=0.10)

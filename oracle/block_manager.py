"""CPU oracle for the block manager: which physical 16-token block holds each
token of each sequence, with prefix sharing, copy on write and swapping.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library never does, and this module imports nothing from it.

What the pages fix:
  - the KV cache is a pool of fixed 16-token physical blocks reached through a
    per-sequence logical block table (LLM Inference Server page, Optional
    Stretch Challenges, "Paged KV-Cache Block Allocator"; Mini inference
    engine page, section 2: a paged allocator with 16-token blocks shared
    across requests);
  - a request whose prompt starts with an already prefilled system prompt
    reuses those K/V blocks and skips prefill on those tokens, with hit/miss
    tracking (LLM Inference Server page, Stage 1 "KV-Cache Engine",
    prefix-cache task; From Scratch page, "Take it further": reuse KV cache
    blocks for shared system prompts across requests);
  - the pool is a fixed budget: a request that does not fit is rejected or
    queued (same Stage 1, footprint-calculator task);
  - the scheduler can preempt a sequence by swapping its blocks out (the
    "preempt/swap" of the Scheduler box, pipeline figure, From Scratch page).

The policy the pages leave open, taken here (and stated the same way in the
library's header):
  1. Free blocks form one FIFO queue, initially 0, 1, ..., n-1.  An allocation
     takes the head; a block whose reference count drops to 0 joins the tail.
     A freed sequence releases its blocks last block first, so that the
     blocks of a common prefix are the last to be reused.
  2. A block that holds tokens stays indexed by (all tokens before it, the
     tokens it holds) until it is reallocated, whether or not a sequence still
     holds it.
  3. A new prompt is matched block by block: among the indexed blocks whose
     preceding tokens equal the prompt's, take the one sharing the longest
     run of leading tokens with the prompt's block (ties: the lowest block id).
     A whole 16-token match continues to the next block; anything shorter
     ends the match.  The match never takes the prompt's last token: that
     token's query row is what produces the first output token, so a prompt
     that is cached whole still prefills its last token.  The matched tokens
     are served from the cache.
  4. Writing a token at offset o of a block the sequence holds: if another
     sequence holds the block too, copy it first (copy on write) to a newly
     allocated block and write there; if the sequence holds it alone and the
     block holds more than o tokens (cached tokens of an earlier owner), those
     are dropped and the token is written in place.
  5. Admission is all or nothing: if the free queue cannot supply every block
     an operation needs, it fails and nothing changes.
  6. Swap out copies every block of the sequence to host blocks (a FIFO queue
     of its own) and releases the device blocks; swap in allocates new device
     blocks and releases the host blocks.

Block content is modelled exactly: no hashing, the index key is the tuple of
preceding tokens itself.
"""
from __future__ import annotations

import math

BLOCK = 16


class NoBlocks(Exception):
    """The operation needs more free blocks than there are; nothing changed."""


class BlockManager:
    def __init__(self, n_blocks: int, n_host_blocks: int = 0, prefix_cache: bool = True):
        self.n_blocks = n_blocks
        self.prefix_cache = prefix_cache
        self.free = list(range(n_blocks))
        self.host_free = list(range(n_host_blocks))
        self.ref = [0] * n_blocks
        self.held = [[] for _ in range(n_blocks)]      # token ids in slots 0..len-1
        self.before = [None] * n_blocks                # tuple of preceding tokens if indexed
        self.seqs = {}
        self.hit_tokens = 0
        self.query_tokens = 0
        self.hit_requests = 0
        self.requests = 0

    # -- blocks ---------------------------------------------------------------
    def _alloc(self) -> int:
        b = self.free.pop(0)
        self.before[b] = None
        self.held[b] = []
        self.ref[b] = 1
        return b

    def _release(self, b: int):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def _claim(self, b: int):
        if self.ref[b] == 0:
            self.free.remove(b)
        self.ref[b] += 1

    def _lookup(self, before: tuple, toks: list):
        best, best_m = None, 0
        for b in range(self.n_blocks):
            if self.before[b] != before:
                continue
            m = 0
            while m < min(len(toks), len(self.held[b])) and self.held[b][m] == toks[m]:
                m += 1
            if m > best_m:
                best, best_m = b, m
        return best, best_m

    # -- the write path (rule 4) ---------------------------------------------
    def _needs(self, seq, n_new: int) -> int:
        """Blocks the free queue must supply to write n_new more tokens."""
        L = len(seq["tokens"])
        fresh = math.ceil((L + n_new) / BLOCK) - len(seq["table"])
        cow = 0
        if n_new and L % BLOCK and self.ref[seq["table"][L // BLOCK]] > 1:
            cow = 1
        return fresh + cow

    def _write(self, seq, toks, slots, pairs):
        for t in toks:
            p = len(seq["tokens"])
            j, o = divmod(p, BLOCK)
            if j == len(seq["table"]):
                seq["table"].append(self._alloc())
            b = seq["table"][j]
            if self.ref[b] > 1:
                d = self._alloc()
                pairs.append((b, d))
                self.held[d] = self.held[b][:o]
                self._release(b)
                seq["table"][j] = b = d
            elif len(self.held[b]) > o:
                self.held[b] = self.held[b][:o]
            self.held[b].append(t)
            if self.prefix_cache:
                self.before[b] = tuple(seq["tokens"][:j * BLOCK])
            seq["tokens"].append(t)
            slots.append(b * BLOCK + o)

    # -- operations -------------------------------------------------------------
    def add_sequence(self, sid, tokens):
        """Admit a prompt.  Returns (n_cached, slots, cow_pairs): slots[i] is
        the slot of token i, -1 for the n_cached leading tokens already in the
        pool."""
        if sid in self.seqs:
            raise KeyError(sid)
        tokens = list(tokens)
        table, pos = [], 0
        if self.prefix_cache:
            # the prompt's last token is never taken from the cache: its query
            # row yields the first output token, so it must be prefilled
            limit = len(tokens) - 1
            while pos < limit:
                b, m = self._lookup(tuple(tokens[:pos]), tokens[pos:min(pos + BLOCK, limit)])
                if m == 0:
                    break
                table.append(b)
                pos += m
                if m < BLOCK:
                    break
        seq = {"table": table, "tokens": tokens[:pos], "swapped": False}
        # admission (rule 5): claimed free blocks plus the blocks the write needs
        from_free = sum(1 for b in table if self.ref[b] == 0)
        fresh = math.ceil(len(tokens) / BLOCK) - len(table)
        cow = 1 if (pos < len(tokens) and pos % BLOCK and self.ref[table[-1]] >= 1) else 0
        if from_free + fresh + cow > len(self.free):
            raise NoBlocks()
        for b in table:
            self._claim(b)
        slots, pairs = [-1] * pos, []
        self._write(seq, tokens[pos:], slots, pairs)
        self.seqs[sid] = seq
        self.requests += 1
        self.query_tokens += len(tokens)
        self.hit_tokens += pos
        self.hit_requests += pos > 0
        return pos, slots, pairs

    def append(self, sid, tokens):
        """Append tokens (a decode step).  Returns (slots, cow_pairs)."""
        seq = self.seqs[sid]
        if seq["swapped"]:
            raise KeyError(sid)
        if self._needs(seq, len(tokens)) > len(self.free):
            raise NoBlocks()
        slots, pairs = [], []
        self._write(seq, list(tokens), slots, pairs)
        return slots, pairs

    def append_batch(self, sids, tokens):
        """One token per sequence, in order, all or nothing.  Returns (slots,
        cow_pairs)."""
        if len(set(sids)) != len(sids):
            raise KeyError("a sequence named twice")
        import copy
        saved = copy.deepcopy(self.__dict__)
        slots, pairs = [], []
        try:
            for sid, t in zip(sids, tokens):
                s, p = self.append(sid, [t])
                slots += s
                pairs += p
        except NoBlocks:
            self.__dict__.update(saved)
            raise
        return slots, pairs

    def fork(self, parent, child):
        p = self.seqs[parent]
        if child in self.seqs or p["swapped"]:
            raise KeyError(child)
        for b in p["table"]:
            self.ref[b] += 1
        self.seqs[child] = {"table": list(p["table"]), "tokens": list(p["tokens"]),
                            "swapped": False}

    def free_sequence(self, sid):
        seq = self.seqs.pop(sid)
        if seq["swapped"]:
            self.host_free.extend(reversed(seq["table"]))
        else:
            for b in reversed(seq["table"]):
                self._release(b)

    def swap_out(self, sid):
        """Returns the (device block, host block) pairs to copy."""
        seq = self.seqs[sid]
        if seq["swapped"]:
            raise KeyError(sid)
        if len(seq["table"]) > len(self.host_free):
            raise NoBlocks()
        host = [self.host_free.pop(0) for _ in seq["table"]]
        pairs = list(zip(seq["table"], host))
        for b in reversed(seq["table"]):
            self._release(b)
        seq["table"], seq["swapped"] = host, True
        return pairs

    def swap_in(self, sid):
        """Returns the (host block, device block) pairs to copy."""
        seq = self.seqs[sid]
        if not seq["swapped"]:
            raise KeyError(sid)
        if len(seq["table"]) > len(self.free):
            raise NoBlocks()
        dev = [self._alloc() for _ in seq["table"]]
        for j, d in enumerate(dev):
            self.held[d] = seq["tokens"][j * BLOCK:(j + 1) * BLOCK]
            if self.prefix_cache:
                self.before[d] = tuple(seq["tokens"][:j * BLOCK])
        pairs = list(zip(seq["table"], dev))
        self.host_free.extend(reversed(seq["table"]))
        seq["table"], seq["swapped"] = dev, False
        return pairs

    def block_table(self, sid):
        seq = self.seqs[sid]
        if seq["swapped"]:
            raise KeyError(sid)
        return list(seq["table"]), len(seq["tokens"])

    def stats(self):
        return {"free": len(self.free), "host_free": len(self.host_free),
                "cached": sum(b is not None for b in self.before),
                "cached_free": sum(self.before[b] is not None for b in self.free),
                "hit_tokens": self.hit_tokens, "query_tokens": self.query_tokens,
                "hit_requests": self.hit_requests, "requests": self.requests}


def kv_cache_bytes(n_layers: int, n_kv_heads: int, d_head: int, batch: int, seq_len: int,
                   bytes_per_elem: int, paged: bool = False) -> int:
    """The KV-cache footprint of the LLM Inference Server page (Required
    Mathematical Concepts): 2 * n_layers * n_kv_heads * d_head * seq_len *
    bytes_per_elem per sequence, times the batch; paged, each sequence's
    length is rounded up to whole 16-token blocks."""
    L = math.ceil(seq_len / BLOCK) * BLOCK if paged else seq_len
    return 2 * n_layers * n_kv_heads * d_head * L * bytes_per_elem * batch

"""Oracle of the steps around the attention path that fill and share the paged
KV cache -- TEST INFRASTRUCTURE ONLY (see the package header).

What is computed
----------------
* **Append.**  Each decode step adds the new tokens' K and V to the cache, and
  later steps reuse them ("vLLM: LLM Inference That Doesn't Waste Your GPU",
  section "KV cache, in one picture").  Token ``t`` of a sequence lives in
  physical block ``block_tables[s, t // B]`` at slot ``t % B``
  ("Local_LLM_03_vLLM_Architecture", PagedAttention slide).  With the
  convention of the attention calls (``context_lens`` already counts the new
  tokens, which are the last ``n_s`` positions), new token ``i`` of sequence
  ``s`` goes to position ``L_s - n_s + i``.
* **Block copies.**  ``copy_blocks`` duplicates whole physical blocks (every
  KV head, every slot).  It serves copy-on-write of a shared block (below).
* **Block pool.**  The cache is a pool of fixed-size blocks handed out on
  demand, so a sequence of ``L`` tokens holds ``ceil(L / B)`` blocks and wastes
  fewer than ``B`` slots ("Scaling inference with vLLM", paging paragraph;
  "vLLM: LLM Inference That Doesn't Waste Your GPU", section "PagedAttention:
  virtual memory for KV").  Requests with a common start physically share the
  pages of that start instead of copying them ("Scaling inference with vLLM",
  prefix-sharing paragraph; "Local_LLM_03_vLLM_Architecture", prefix-caching
  slide).  ``BlockPoolModel`` states these rules; the pages say nothing of how
  shared pages are released or written, so the model takes the plain reading:
  a block carries a count of the tables that hold it and returns to the free
  set when that count reaches zero; a sequence that appends into a partially
  filled block that other tables also hold first gets a private copy of it
  (copy-on-write), while a full shared block is never written again.  Which
  free block is handed out is the allocator's choice; the model picks the
  lowest id, and tests compare only what does not depend on that choice.
* **Prefix caching.**  The pages' server hashes each page's token content, and
  two requests with the same first ``N`` tokens share ``N / B`` physical pages
  with no recomputation ("Local_LLM_03_vLLM_Architecture", prefix-caching
  slide; "vLLM: LLM Inference That Doesn't Waste Your GPU", section "Prefix
  caching").  The model keys a full block by the exact tokens from the start
  of the sequence to the end of that block (the plain meaning of "the same
  first N tokens"): ``commit`` registers a sequence's full blocks once their
  K/V are written, ``match_prefix`` gives an empty sequence every leading
  full block already registered under the same token prefix.  A block leaves
  the cache when it returns to the free set.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


def append_kv(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              block_tables: np.ndarray, context_lens: np.ndarray, q_offsets: np.ndarray,
              block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the pools with every new token's K/V written into its slot.

    ``k_new``/``v_new``: ``[total_new, Hk, D]``; the new tokens of sequence ``s``
    are rows ``q_offsets[s]:q_offsets[s+1]`` and take positions
    ``L_s - n_s .. L_s - 1``.  Bytes are moved unchanged.
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    for s in range(len(context_lens)):
        q0, q1 = int(q_offsets[s]), int(q_offsets[s + 1])
        n, L = q1 - q0, int(context_lens[s])
        for i in range(n):
            t = L - n + i
            b = int(block_tables[s, t // block_size])
            kc[b, :, t % block_size, :] = k_new[q0 + i]
            vc[b, :, t % block_size, :] = v_new[q0 + i]
    return kc, vc


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray,
                pairs: Sequence[Tuple[int, int]]) -> Tuple[np.ndarray, np.ndarray]:
    """Copies of the pools where block ``dst`` holds what block ``src`` held, for
    every ``(src, dst)`` pair.  Destinations are distinct and are never a source,
    so the copies do not depend on their order."""
    dsts = [d for _, d in pairs]
    assert len(set(dsts)) == len(dsts) and not set(dsts) & {s for s, _ in pairs}
    kc, vc = k_cache.copy(), v_cache.copy()
    for src, dst in pairs:
        kc[dst] = k_cache[src]
        vc[dst] = v_cache[src]
    return kc, vc


class OutOfBlocks(Exception):
    pass


class BlockPoolModel:
    """Reference model of a paged block pool with shared blocks and copy-on-write."""

    def __init__(self, num_blocks: int, block_size: int):
        self.B = block_size
        self.free = set(range(num_blocks))
        self.ref: Dict[int, int] = {}
        self.blocks: Dict[int, List[int]] = {}
        self.length: Dict[int, int] = {}
        self._next_seq = 0
        self.cached: Dict[tuple, int] = {}      # token prefix through a full block -> block

    def _take(self) -> int:
        b = min(self.free)
        self.free.remove(b)
        self.ref[b] = 1
        return b

    def _drop(self, b: int):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            del self.ref[b]
            self.free.add(b)
            self.cached = {k: v for k, v in self.cached.items() if v != b}

    def create(self) -> int:
        s = self._next_seq
        self._next_seq += 1
        self.blocks[s], self.length[s] = [], 0
        return s

    def fork(self, parent: int) -> int:
        """A new sequence holding the parent's blocks (a shared prefix)."""
        s = self.create()
        self.blocks[s] = list(self.blocks[parent])
        self.length[s] = self.length[parent]
        for b in self.blocks[s]:
            self.ref[b] += 1
        return s

    def release(self, s: int):
        for b in self.blocks.pop(s):
            self._drop(b)
        del self.length[s]

    def append(self, s: int, n: int) -> List[Tuple[int, int]]:
        """Grow sequence ``s`` by ``n`` tokens; returns the (src, dst) block copies
        that must run before the new tokens are written.  All or nothing."""
        L, B = self.length[s], self.B
        if n == 0:
            return []
        cow = L % B != 0 and self.ref[self.blocks[s][-1]] > 1
        need = -(-(L + n) // B) - -(-L // B) + (1 if cow else 0)
        if need > len(self.free):
            raise OutOfBlocks()
        pairs = []
        if cow:
            old = self.blocks[s][-1]
            new = self._take()
            pairs.append((old, new))
            self.blocks[s][-1] = new
            self._drop(old)
        while len(self.blocks[s]) < -(-(L + n) // B):
            self.blocks[s].append(self._take())
        self.length[s] = L + n
        return pairs

    def match_prefix(self, s: int, tokens: Sequence[int]) -> int:
        """Point the empty sequence ``s`` at every leading full block registered
        under the same token prefix; returns the number of tokens it now holds."""
        assert self.length[s] == 0
        B, j = self.B, 0
        while (j + 1) * B <= len(tokens):
            b = self.cached.get(tuple(tokens[:(j + 1) * B]))
            if b is None:
                break
            self.blocks[s].append(b)
            self.ref[b] += 1
            j += 1
        self.length[s] = j * B
        return j * B

    def commit(self, s: int, tokens: Sequence[int]) -> int:
        """Register the full blocks of ``s`` among its first ``len(tokens)`` tokens
        (whose K/V are written); a prefix already registered keeps its block.
        Returns how many blocks were newly registered."""
        assert len(tokens) <= self.length[s]
        new = 0
        for j in range(len(tokens) // self.B):
            key = tuple(tokens[:(j + 1) * self.B])
            if key not in self.cached:
                self.cached[key] = self.blocks[s][j]
                new += 1
        return new

    def num_free(self) -> int:
        return len(self.free)

    def table(self, s: int) -> List[int]:
        return list(self.blocks[s])

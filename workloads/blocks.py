"""Host block manager with reference counts: a generator of multi-step
decode workloads in which sequences share blocks and copy them on write.

This module draws inputs and builds structure only (block tables, slots,
copy pairs, new-token values); it computes none of the attention, copy or
write arithmetic, so both the CPU oracle side and the GPU side of a test can
take their inputs from it.

The manager follows the pages' allocator:
* adg.csdn.net article on ATB's KV Cache management, "BlockManager 的调度":
  a free list of physical blocks, ceil(tokens / 16) blocks per sequence,
  one more block when a sequence crosses a block boundary, blocks returned
  when a sequence finishes;
* zskr.cn article on ATB's PagedAttention, "踩坑二": a block shared by
  several sequences carries a reference count and is freed only at zero;
  "踩坑三": before a token is written into a block another sequence still
  references, the writer takes a fresh block and the old contents are
  copied into it (copy-on-write).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 16


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, rng: np.random.Generator | None = None):
        self.num_blocks = int(num_blocks)
        order = np.arange(self.num_blocks)
        if rng is not None:
            order = rng.permutation(self.num_blocks)     # scattered physical placement
        self.free = [int(b) for b in order[::-1]]        # pop() takes order[0] first
        self.ref = np.zeros(self.num_blocks, dtype=np.int64)
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}

    # -- allocation ----------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise OutOfBlocks("no free block")
        b = self.free.pop()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _drop(self, b: int) -> None:
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0:
            self.free.append(b)

    def allocate(self, seq: int, num_tokens: int) -> list[int]:
        """A new sequence whose first num_tokens tokens (its prompt) are
        already cached: ceil(num_tokens / 16) fresh blocks."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        n = -(-int(num_tokens) // BLOCK)
        self.tables[seq] = [self._take() for _ in range(n)]
        self.lens[seq] = int(num_tokens)
        return list(self.tables[seq])

    def fork(self, parent: int, child: int) -> None:
        """child starts as a copy of parent sharing every block (parallel
        sampling, beam search, a shared prompt)."""
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append_slot(self, seq: int) -> tuple[int, tuple[int, int] | None]:
        """Slot of seq's next token, and the (src, dst) block copy that must
        run before the token is written, if any."""
        table = self.tables[seq]
        L = self.lens[seq]
        copy = None
        if L % BLOCK == 0:                   # no room left: a fresh block
            table.append(self._take())
        elif self.ref[table[-1]] > 1:        # shared partial block: copy on write
            old = table[-1]
            new = self._take()
            copy = (old, new)
            self._drop(old)
            table[-1] = new
        self.lens[seq] = L + 1
        return table[L // BLOCK] * BLOCK + L % BLOCK, copy

    def release(self, seq: int) -> None:
        for b in self.tables.pop(seq):
            self._drop(b)
        del self.lens[seq]

    # -- views -----------------------------------------------------------------
    def check(self) -> None:
        """Reference counts equal table references; free blocks have none."""
        count = np.zeros(self.num_blocks, dtype=np.int64)
        for t in self.tables.values():
            for b in t:
                count[b] += 1
        assert np.array_equal(count, self.ref)
        assert sorted(self.free) == sorted(np.flatnonzero(self.ref == 0).tolist())
        for seq, t in self.tables.items():
            assert len(t) == -(-self.lens[seq] // BLOCK)

    def block_table(self, seqs: list[int], width: int | None = None) -> np.ndarray:
        width = width or max(len(self.tables[s]) for s in seqs)
        bt = np.zeros((len(seqs), width), dtype=np.int32)
        for i, s in enumerate(seqs):
            bt[i, :len(self.tables[s])] = self.tables[s]
        return bt


@dataclass
class Step:
    seqs: list[int]                  # sequences decoded this step, in batch order
    pairs: np.ndarray                # int32 [n, 2] copy-on-write (src, dst)
    slots: np.ndarray                # int32 [B] slot of each sequence's new token
    k_new: np.ndarray                # fp16 [B, Hkv, D]
    v_new: np.ndarray
    q: np.ndarray                    # fp16 [B, Hq, D]
    block_table: np.ndarray          # int32 [B, width]
    context_lens: np.ndarray         # int32 [B], including the new token


@dataclass
class Scenario:
    num_blocks: int
    kv_heads: int
    head_dim: int
    q_heads: int
    steps: list[Step] = field(default_factory=list)


def cow_scenario(seed: int = 0, *, num_blocks: int = 96, kv_heads: int = 2, head_dim: int = 64,
                 q_heads: int = 4, steps: int = 24) -> Scenario:
    """Decode steps over sequences that fork from one another mid-block, so
    that copy-on-write happens, some finish and free their blocks, and new
    sequences reuse them.  Values are seeded N(0,1) fp16."""
    rng = np.random.default_rng(seed)
    bm = BlockManager(num_blocks, rng)
    sc = Scenario(num_blocks, kv_heads, head_dim, q_heads)
    next_id = 0

    def new_seq(n):
        nonlocal next_id
        bm.allocate(next_id, n)
        next_id += 1
        return next_id - 1

    live = [new_seq(int(rng.integers(5, 60))) for _ in range(3)]
    for step in range(steps):
        # occasionally fork a live sequence (its partial last block becomes shared)
        if rng.random() < 0.4 and len(live) < 8:
            parent = live[int(rng.integers(len(live)))]
            bm.fork(parent, next_id)
            live.append(next_id)
            next_id += 1
        # occasionally finish one and start a fresh one
        if rng.random() < 0.2 and len(live) > 2:
            bm.release(live.pop(int(rng.integers(len(live)))))
            live.append(new_seq(int(rng.integers(1, 40))))
        pairs, slots = [], []
        for s in live:
            slot, copy = bm.append_slot(s)
            slots.append(slot)
            if copy is not None:
                pairs.append(copy)
        bm.check()
        B = len(live)
        sc.steps.append(Step(
            seqs=list(live),
            pairs=np.array(pairs, dtype=np.int32).reshape(-1, 2),
            slots=np.array(slots, dtype=np.int32),
            k_new=rng.standard_normal((B, kv_heads, head_dim), dtype=np.float32).astype(np.float16),
            v_new=rng.standard_normal((B, kv_heads, head_dim), dtype=np.float32).astype(np.float16),
            q=rng.standard_normal((B, q_heads, head_dim), dtype=np.float32).astype(np.float16),
            block_table=bm.block_table(live),
            context_lens=np.array([bm.lens[s] for s in live], dtype=np.int32),
        ))
    return sc

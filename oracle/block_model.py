"""Dictionary model of the KV block manager.

TEST INFRASTRUCTURE ONLY (see the package docstring): the reference for the host
block manager in ``paged_kv_cache_76_amd.block_manager``; it shares no code
with it.

Sources:

* "vLLM / PagedAttention" (awesome.papernotes.org), "方法详解":
  key design 2 — each sequence's logical blocks record a physical id and a
  filled count; prefill allocates enough blocks for the prompt; each decoded
  token goes into the last block and a new physical block is allocated when
  that block is full.  Key design 3 — physical blocks carry reference counts;
  a write into a shared block (count > 1) allocates a new block, copies the
  old content into it, decrements the old count and remaps the logical block;
  the ``append_token`` pseudocode fixes the order of those checks (full first,
  then shared).
* "vLLM" notes (formulaic.cloudchewie.com), "PagedAttention 原理" (7-token
  prompt with B=4 → two blocks filled 4 and 3, the first decoded token fills
  the second block, the next one opens a third) and "Parallel Sampling 场景"
  (two samples share two physical blocks with count 2; the first sample's
  write copies the shared partial block into a new one; afterwards the
  counts are 1, 1 and 2).
* "vLLM / PagedAttention (SOSP 2023)" guide, section 03 (a new block is
  allocated only when all previous ones are full; a finished request's blocks
  are released), section 04 (fork shares blocks; copy-on-write copies one
  block).

Readings taken where the pages are silent or disagree:

* Allocation is lazy: the block for token ``k*B`` is allocated when that token
  is appended (key design 3's pseudocode and section 03), not eagerly when
  the previous block fills (the cloudchewie walk-through).  Only the lazy
  reading keeps the strict tail bound ``w_tail < B * s_kv`` of key design 2.
* A full *and* shared last block gets a fresh block and no copy, because the
  pseudocode tests ``is_full`` first.
* Physical ids come from a free list: allocation takes the front, release
  appends to the back; the initial order is an input (a seeded permutation).
  Releasing a sequence releases its blocks in logical order.
* Within one decode step sequences append in ascending order, so the first
  writer of a shared block copies and the last sharer writes in place.
"""

from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field


class OutOfBlocks(RuntimeError):
    """The free list is empty."""


@dataclass
class LogicalBlock:
    physical: int
    filled: int


@dataclass
class Sequence:
    blocks: list = field(default_factory=list)   # list[LogicalBlock]

    @property
    def length(self) -> int:
        return sum(b.filled for b in self.blocks)


class BlockModel:
    """Reference block manager: free list, reference counts, block tables,
    lazy append, fork, free and copy-on-write, one token at a time."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if block_size < 1 or num_blocks < 0:
            raise ValueError("block_size >= 1 and num_blocks >= 0 are required")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self.B = block_size
        self.num_blocks = num_blocks
        self.free_list = deque(order)
        self.ref: dict[int, int] = {}
        self.seqs: dict[int, Sequence] = {}
        self.copies: list[tuple[int, int]] = []   # every (src, dst) ever emitted

    # -- physical blocks --------------------------------------------------
    def _allocate(self) -> int:
        if not self.free_list:
            raise OutOfBlocks("no free physical block")
        phys = self.free_list.popleft()
        self.ref[phys] = 1
        return phys

    def _release(self, phys: int) -> None:
        if self.ref.get(phys, 0) <= 0:
            raise RuntimeError(f"release of unreferenced block {phys}")
        self.ref[phys] -= 1
        if self.ref[phys] == 0:
            del self.ref[phys]
            self.free_list.append(phys)

    # -- sequence operations ----------------------------------------------
    def add_prompt(self, sid: int, length: int) -> list[int]:
        """Allocate ceil(length/B) blocks for a prompt; return its slots."""
        if sid in self.seqs:
            raise KeyError(f"sequence {sid} exists")
        if length < 1:
            raise ValueError("a prompt has at least one token")
        n = -(-length // self.B)
        if n > len(self.free_list):
            raise OutOfBlocks(f"prompt needs {n} blocks, {len(self.free_list)} free")
        seq = Sequence()
        for j in range(n):
            filled = self.B if j < n - 1 else length - (n - 1) * self.B
            seq.blocks.append(LogicalBlock(self._allocate(), filled))
        self.seqs[sid] = seq
        return [self.slot(sid, p) for p in range(length)]

    def append(self, sid: int) -> tuple[int, tuple[int, int] | None]:
        """Append one token (key design 3, ``append_token``).

        Returns the slot the token's K/V go to and the ``(src, dst)`` copy the
        write needs first, or ``None``.
        """
        seq = self.seqs[sid]
        last = seq.blocks[-1]
        pair = None
        if last.filled == self.B:
            last = LogicalBlock(self._allocate(), 0)
            seq.blocks.append(last)
        elif self.ref[last.physical] > 1:
            new = self._allocate()
            pair = (last.physical, new)
            self.copies.append(pair)
            self.ref[last.physical] -= 1
            last.physical = new
        slot = last.physical * self.B + last.filled
        last.filled += 1
        return slot, pair

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent (counts + 1)."""
        if child in self.seqs:
            raise KeyError(f"sequence {child} exists")
        src = self.seqs[parent]
        self.seqs[child] = Sequence([LogicalBlock(b.physical, b.filled) for b in src.blocks])
        for b in src.blocks:
            self.ref[b.physical] += 1

    def free(self, sid: int) -> None:
        """Release every block of a sequence, in logical order."""
        seq = self.seqs.pop(sid)
        for b in seq.blocks:
            self._release(b.physical)

    # -- views ------------------------------------------------------------
    def table(self, sid: int) -> list[int]:
        return [b.physical for b in self.seqs[sid].blocks]

    def filled(self, sid: int) -> list[int]:
        return [b.filled for b in self.seqs[sid].blocks]

    def length(self, sid: int) -> int:
        return self.seqs[sid].length

    def slot(self, sid: int, pos: int) -> int:
        """Physical slot of logical position ``pos`` of a sequence."""
        b = self.seqs[sid].blocks[pos // self.B]
        return b.physical * self.B + pos % self.B

    def used(self) -> int:
        return len(self.ref)

    def tail_waste(self, sid: int) -> int:
        """Unused slots of the sequence's blocks (key design 2, eq. 3, in
        tokens): ``len(table) * B - L``."""
        return len(self.seqs[sid].blocks) * self.B - self.length(sid)

    def check_invariants(self) -> None:
        """Raise ``AssertionError`` if the state is inconsistent."""
        counts: dict[int, int] = {}
        for sid, seq in self.seqs.items():
            ids = [b.physical for b in seq.blocks]
            assert len(ids) == len(set(ids)), f"seq {sid} maps one block twice"
            assert seq.blocks, f"seq {sid} has no block"
            assert all(b.filled == self.B for b in seq.blocks[:-1]), f"seq {sid}: a non-last block is not full"
            assert 1 <= seq.blocks[-1].filled <= self.B, f"seq {sid}: bad filled count"
            L = seq.length
            assert len(ids) == -(-L // self.B)
            assert 0 <= self.tail_waste(sid) <= self.B - 1
            for i in ids:
                counts[i] = counts.get(i, 0) + 1
        assert counts == self.ref, "reference counts differ from table references"
        free = set(self.free_list)
        assert len(free) == len(self.free_list), "a block is free twice"
        assert not (free & set(self.ref)), "a block is both free and used"
        assert free | set(self.ref) == set(range(self.num_blocks)), "a block is lost"
        # key design 3, eq. 4 made exact: every extra reference is one block saved
        logical = sum(len(s.blocks) for s in self.seqs.values())
        shared = sum(c - 1 for c in self.ref.values())
        assert logical - shared == self.used()

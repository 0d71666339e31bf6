"""Host-side KV block manager: free list, reference counts, lazy append,
fork, free and copy-on-write, producing the device-ready block tables, slot
mappings and copy pairs that the kernels consume.

Sources: "vLLM / PagedAttention" (awesome.papernotes.org), "方法详解"
key design 2 (each sequence's logical blocks map to physical blocks through a
block table; prefill allocates the prompt's blocks, each decoded token goes
into the last block, a new block is allocated when that one is full) and key
design 3 (reference counts per physical block; a write into a shared block
allocates, copies, decrements and remaps — the ``append_token`` order of
checks: full first, then shared); "vLLM" notes (formulaic.cloudchewie.com),
"PagedAttention 原理" and "在不同解码策略下的效果" (parallel sampling shares
prompt blocks; beam search forks candidates and releases pruned ones);
"vLLM / PagedAttention (SOSP 2023)" guide, sections 03-04.

Design: state is kept in flat numpy arrays indexed by *row* — the sequence's
position in the decode batch — so ``tables`` is already the ``[S][max_blocks]``
int32 array the decode kernel reads, and a decode step over many rows is a
handful of vectorised operations.  Only rows whose last block is shared take
a Python-level path (the copy-on-write decision is sequential by nature: the
i-th appending sharer of a block sees its count lowered by i).

Policies (readings of points the pages leave open):

* lazy allocation: a block is allocated when the token that needs it arrives;
* a full and shared last block gets a fresh block and no copy;
* the free list is FIFO: allocation takes the front, release appends to the
  back; the initial order is an input (a seeded permutation);
* within a step rows append in ascending order, so the first writer of a
  shared block copies and the last sharer writes in place; allocations of a
  step are handed out in ascending row order;
* a step is all-or-nothing: if the free list cannot cover it, nothing changes
  and :class:`OutOfBlocks` is raised;
* slot = physical_id * B + offset (int64); unused table entries hold
  ``poison`` (default: ``num_blocks``, outside the pool).
"""

from __future__ import annotations

import numpy as np


class OutOfBlocks(RuntimeError):
    """The free list cannot cover the request."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, max_rows: int, max_blocks_per_seq: int,
                 free_order=None, poison: int | None = None, host_blocks: int = 0):
        if block_size < 1 or num_blocks < 1:
            raise ValueError("num_blocks and block_size must be >= 1")
        if not 0 <= host_blocks <= num_blocks:
            # the swap space in CPU RAM is bounded by the device memory given
            # to the KV cache ("vLLM / PagedAttention (SOSP 2023)" guide,
            # section 05): at most one host block per device block
            raise ValueError(f"host_blocks = {host_blocks} must lie in [0, num_blocks = {num_blocks}]")
        self.num_blocks = int(num_blocks)
        self.B = int(block_size)
        self.max_rows = int(max_rows)
        self.max_blocks = int(max_blocks_per_seq)
        self.poison = self.num_blocks if poison is None else int(poison)
        order = np.arange(num_blocks, dtype=np.int64) if free_order is None else np.asarray(free_order, np.int64)
        if order.shape != (num_blocks,) or not np.array_equal(np.sort(order), np.arange(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        # FIFO ring of free ids
        self._ring = order.copy()
        self._head = 0
        self._nfree = num_blocks
        self.ref = np.zeros(num_blocks, dtype=np.int32)
        self.tables = np.full((max_rows, max_blocks_per_seq), self.poison, dtype=np.int32)
        self.nblocks = np.zeros(max_rows, dtype=np.int32)
        self.lens = np.zeros(max_rows, dtype=np.int64)
        self.cow_copies = 0
        # host (swap) pool: FIFO free list, reference counts, swapped rows
        self.host_blocks = int(host_blocks)
        self._host_free = list(range(self.host_blocks))
        self.host_ref = np.zeros(self.host_blocks, dtype=np.int32)
        self.swapped: dict[int, tuple[np.ndarray, int]] = {}   # row -> (host ids, length)

    # ---- free list ----------------------------------------------------------
    @property
    def num_free(self) -> int:
        return self._nfree

    def _pop(self, k: int) -> np.ndarray:
        if k > self._nfree:
            raise OutOfBlocks(f"{k} blocks needed, {self._nfree} free")
        idx = (self._head + np.arange(k)) % self.num_blocks
        ids = self._ring[idx].copy()
        self._head = (self._head + k) % self.num_blocks
        self._nfree -= k
        return ids

    def _push(self, ids: np.ndarray) -> None:
        k = len(ids)
        if k == 0:
            return
        tail = (self._head + self._nfree) % self.num_blocks
        self._ring[(tail + np.arange(k)) % self.num_blocks] = ids
        self._nfree += k

    def free_list(self) -> list[int]:
        idx = (self._head + np.arange(self._nfree)) % self.num_blocks
        return self._ring[idx].tolist()

    # ---- sequence operations ------------------------------------------------
    def _check_row(self, row: int, live: bool) -> None:
        if not 0 <= row < self.max_rows:
            raise IndexError(f"row {row} outside [0, {self.max_rows})")
        if row in self.swapped:
            raise KeyError(f"row {row} is swapped out")
        if live and self.lens[row] == 0:
            raise KeyError(f"row {row} holds no sequence")
        if not live and self.lens[row] != 0:
            raise KeyError(f"row {row} already holds a sequence")

    def add_prompt(self, row: int, length: int) -> np.ndarray:
        """Allocate ceil(length/B) blocks for a prompt in ``row``; return the
        int64 slots of its tokens in logical order."""
        self._check_row(row, live=False)
        if length < 1:
            raise ValueError("a prompt has at least one token")
        n = -(-int(length) // self.B)
        if n > self.max_blocks:
            raise ValueError(f"prompt of {length} tokens needs {n} > {self.max_blocks} table entries")
        ids = self._pop(n)
        self.tables[row, :n] = ids
        self.ref[ids] = 1
        self.nblocks[row] = n
        self.lens[row] = length
        pos = np.arange(length, dtype=np.int64)
        return ids[pos // self.B] * self.B + pos % self.B

    def append_step(self, rows) -> tuple[np.ndarray, np.ndarray]:
        """Append one token to each of ``rows`` (processed in ascending order).

        Returns ``(slot_mapping int64 [len(rows)], copy_pairs int64 [P][2])``;
        ``slot_mapping[i]`` belongs to ``sorted(rows)[i]``.  The copies must be
        executed before the new tokens are written.
        """
        rows = np.sort(np.asarray(rows, dtype=np.int64))
        if len(rows) == 0:
            return np.zeros(0, np.int64), np.zeros((0, 2), np.int64)
        if len(np.unique(rows)) != len(rows):
            raise ValueError("a row appears twice in one step")
        if np.any(self.lens[rows] == 0):
            raise KeyError("append to an empty row")
        L = self.lens[rows]
        nb = self.nblocks[rows].astype(np.int64)
        off = L % self.B
        need_new = off == 0                                   # last block full
        if np.any(need_new & (nb >= self.max_blocks)):
            raise ValueError("a sequence outgrew max_blocks_per_seq")
        last = self.tables[rows, nb - 1].astype(np.int64)
        # copy-on-write decision for rows whose partial last block is shared
        cow = np.zeros(len(rows), dtype=bool)
        cand = np.nonzero(~need_new & (self.ref[last] > 1))[0]
        if len(cand):
            seen: dict[int, int] = {}
            for i in cand:                                    # ascending rows
                b = int(last[i])
                k = seen.get(b, 0)
                cow[i] = self.ref[b] - k > 1
                seen[b] = k + 1
        alloc = need_new | cow
        n_alloc = int(alloc.sum())
        ids = self._pop(n_alloc)                              # raises before any change
        new_ids = np.full(len(rows), -1, dtype=np.int64)
        new_ids[alloc] = ids
        # fresh blocks for full last blocks
        r_new = rows[need_new]
        self.tables[r_new, nb[need_new]] = new_ids[need_new]
        self.nblocks[r_new] += 1
        # copy-on-write: remap the last logical block, move one reference
        r_cow = rows[cow]
        src = last[cow]
        self.tables[r_cow, nb[cow] - 1] = new_ids[cow]
        np.subtract.at(self.ref, src, 1)
        self.ref[ids] = 1
        self.cow_copies += int(cow.sum())
        phys = np.where(alloc, new_ids, last)
        slots = phys * self.B + off
        self.lens[rows] += 1
        pairs = np.stack([src, new_ids[cow]], axis=1) if len(src) else np.zeros((0, 2), np.int64)
        return slots.astype(np.int64), pairs.astype(np.int64)

    def extend(self, row: int, n: int) -> tuple[np.ndarray, np.ndarray]:
        """Append ``n`` tokens to one row at once (the same outcome as ``n``
        single appends): returns the tokens' slots and the copy pairs.

        Used for a request that maps a cached prefix and then writes its own
        task input ("vLLM / PagedAttention (SOSP 2023)" guide, section 04:
        the last prefix block is copy-on-write)."""
        self._check_row(row, live=True)
        if n <= 0:
            return np.zeros(0, np.int64), np.zeros((0, 2), np.int64)
        L = int(self.lens[row])
        nb = int(self.nblocks[row])
        off = L % self.B
        room = (self.B - off) % self.B          # free slots in the last block
        new_blocks = -(-(n - room) // self.B) if n > room else 0
        last = int(self.tables[row, nb - 1])
        cow = room > 0 and self.ref[last] > 1    # the first token lands in a shared partial block
        if nb + new_blocks > self.max_blocks:
            raise ValueError("a sequence outgrew max_blocks_per_seq")
        ids = self._pop(new_blocks + int(cow))   # raises before any change
        pairs = np.zeros((0, 2), np.int64)
        if cow:
            copy = int(ids[0])
            pairs = np.array([[last, copy]], np.int64)
            self.ref[last] -= 1
            self.ref[copy] = 1
            self.tables[row, nb - 1] = copy
            self.cow_copies += 1
            last = copy
            ids = ids[1:]
        self.tables[row, nb:nb + new_blocks] = ids
        self.ref[ids] = 1
        self.nblocks[row] = nb + new_blocks
        self.lens[row] = L + n
        pos = np.arange(L, L + n, dtype=np.int64)
        table = self.tables[row, : nb + new_blocks].astype(np.int64)
        return table[pos // self.B] * self.B + pos % self.B, pairs

    def fork(self, src_row: int, dst_row: int) -> None:
        """``dst_row`` shares every block of ``src_row`` (counts + 1)."""
        self._check_row(src_row, live=True)
        self._check_row(dst_row, live=False)
        n = int(self.nblocks[src_row])
        ids = self.tables[src_row, :n]
        self.tables[dst_row, :n] = ids
        self.ref[ids] += 1
        self.nblocks[dst_row] = n
        self.lens[dst_row] = self.lens[src_row]

    def free(self, row: int) -> None:
        """Release every block of ``row`` in logical order."""
        self._check_row(row, live=True)
        n = int(self.nblocks[row])
        ids = self.tables[row, :n].astype(np.int64)
        self.ref[ids] -= 1
        self._push(ids[self.ref[ids] == 0])
        self.tables[row, :] = self.poison
        self.nblocks[row] = 0
        self.lens[row] = 0

    # ---- swapping (preemption) ----------------------------------------------
    def swap_out(self, rows) -> np.ndarray:
        """Evict a group of rows all-or-nothing: every distinct block they map
        moves to the host pool ("vLLM" notes, 调度和抢占; the SOSP guide,
        section 05).  Returns (device, host) pairs for ``pa_swap_blocks``;
        the copies must run before the freed device blocks are reused.  A
        block shared inside the group stays shared on the host."""
        rows = sorted(set(int(r) for r in rows))
        for r in rows:
            self._check_row(r, live=True)
        dev = []
        seen = set()
        for r in rows:
            for b in self.tables[r, : self.nblocks[r]].tolist():
                if b not in seen:
                    seen.add(b)
                    dev.append(b)
        if len(dev) > len(self._host_free):
            raise OutOfBlocks(f"{len(dev)} host blocks needed, {len(self._host_free)} free")
        host = [self._host_free.pop(0) for _ in dev]
        to_host = dict(zip(dev, host))
        for r in rows:
            ids = self.tables[r, : self.nblocks[r]].astype(np.int64)
            hids = np.array([to_host[int(b)] for b in ids], dtype=np.int64)
            self.host_ref[hids] += 1
            self.swapped[r] = (hids, int(self.lens[r]))
            self.ref[ids] -= 1
            self._push(ids[self.ref[ids] == 0])
            self.tables[r, :] = self.poison
            self.nblocks[r] = 0
            self.lens[r] = 0
        return np.array([[d, h] for d, h in zip(dev, host)], dtype=np.int64).reshape(-1, 2)

    def swap_in(self, rows) -> np.ndarray:
        """Bring swapped rows back: one fresh device block per distinct host
        block.  Returns (host, device) pairs for ``pa_swap_blocks``."""
        rows = sorted(set(int(r) for r in rows))
        for r in rows:
            if r not in self.swapped:
                raise KeyError(f"row {r} is not swapped out")
        hosts = []
        seen = set()
        for r in rows:
            for h in self.swapped[r][0].tolist():
                if h not in seen:
                    seen.add(h)
                    hosts.append(h)
        ids = self._pop(len(hosts))              # raises before any change
        to_dev = dict(zip(hosts, ids.tolist()))
        for r in rows:
            hids, length = self.swapped.pop(r)
            dev = np.array([to_dev[int(h)] for h in hids], dtype=np.int64)
            self.tables[r, : len(dev)] = dev
            self.nblocks[r] = len(dev)
            self.lens[r] = length
            np.add.at(self.ref, dev, 1)
            self.host_ref[hids] -= 1
        for h in hosts:
            if self.host_ref[h] == 0:
                self._host_free.append(h)
        return np.array([[h, to_dev[h]] for h in hosts], dtype=np.int64).reshape(-1, 2)

    # ---- views and accounting -------------------------------------------------
    def table(self, row: int) -> list[int]:
        return self.tables[row, : self.nblocks[row]].tolist()

    def slot(self, row: int, pos: int) -> int:
        return int(self.tables[row, pos // self.B]) * self.B + pos % self.B

    def live_rows(self) -> np.ndarray:
        return np.nonzero(self.lens > 0)[0]

    def used(self) -> int:
        return int(np.count_nonzero(self.ref))

    def tail_waste(self, rows=None) -> np.ndarray:
        """Unused slots in each row's blocks (key design 2, eq. 3, in tokens)."""
        rows = self.live_rows() if rows is None else np.asarray(rows)
        return self.nblocks[rows].astype(np.int64) * self.B - self.lens[rows]

    def blocks_saved_by_sharing(self) -> int:
        """Extra references (key design 3, eq. 4): logical - physical blocks."""
        r = self.ref[self.ref > 0]
        return int((r - 1).sum())

    def stats(self) -> dict:
        live = self.live_rows()
        waste = self.tail_waste(live)
        hist = np.bincount(self.ref[self.ref > 0]) if self.used() else np.zeros(1, np.int64)
        return {
            "live_sequences": int(len(live)),
            "used_blocks": self.used(),
            "free_blocks": self.num_free,
            "logical_blocks": int(self.nblocks[live].sum()),
            "blocks_saved_by_sharing": self.blocks_saved_by_sharing(),
            "tokens": int(self.lens[live].sum()),
            "tail_waste_slots": int(waste.sum()),
            "slot_utilisation": float(self.lens[live].sum() / max(1, self.used() * self.B)),
            "ref_count_histogram": {int(k): int(v) for k, v in enumerate(hist) if k > 0 and v},
            "cow_copies": self.cow_copies,
        }


class PrefixCache:
    """A provider's set of predefined prefixes kept in reserved physical
    blocks ("vLLM / PagedAttention (SOSP 2023)" guide, section 04: the
    provider reserves blocks for a set of prefixes; a request whose prompt
    starts with one of them maps those blocks and computes only its own task
    input, the last prefix block being copy-on-write).

    Each registered prefix holds its blocks through a row of the block
    manager reserved for it (one reference per block).  ``attach`` maps a
    prefix into a request's row (a fork: every prefix block gains a
    reference) and extends the row by the request's task tokens; a task
    token landing in a partial, shared last prefix block first copies that
    block (``extend``'s copy-on-write pair).  ``release`` drops the
    provider's references: blocks still mapped by requests stay until those
    requests are freed, then return to the free list.
    """

    def __init__(self, mgr: BlockManager, rows):
        self.mgr = mgr
        self._spare = sorted(int(r) for r in rows)   # rows reserved for prefixes, unused
        self._row: dict[str, int] = {}                # prefix name -> its row
        self.hits: dict[str, int] = {}                # requests attached to each prefix

    @property
    def names(self) -> list[str]:
        return sorted(self._row)

    def row(self, name: str) -> int:
        if name not in self._row:
            raise KeyError(f"no prefix named {name!r}")
        return self._row[name]

    def register(self, name: str, length: int) -> np.ndarray:
        """Reserve blocks for a prefix of ``length`` tokens; returns the int64
        slots its keys/values go to (write them with pa_reshape_and_cache
        before any request attaches)."""
        if name in self._row:
            raise KeyError(f"prefix {name!r} is already registered")
        if not self._spare:
            raise RuntimeError("no row left for another prefix")
        row = self._spare[0]
        slots = self.mgr.add_prompt(row, length)      # raises OutOfBlocks before any change
        self._spare.pop(0)
        self._row[name] = row
        self.hits[name] = 0
        return slots

    def attach(self, name: str, row: int, task_len: int) -> tuple[np.ndarray, np.ndarray]:
        """Map prefix ``name`` into the empty ``row`` and extend it by
        ``task_len`` tokens.  Returns the task tokens' slots and the
        copy-on-write pairs to run (pa_copy_blocks) before writing them."""
        src = self.row(name)
        self.mgr.fork(src, row)
        try:
            slots, pairs = self.mgr.extend(row, task_len)
        except Exception:
            self.mgr.free(row)                        # undo the fork: all-or-nothing
            raise
        self.hits[name] += 1
        return slots, pairs

    def release(self, name: str) -> None:
        """Drop the provider's references to a prefix's blocks."""
        row = self.row(name)
        self.mgr.free(row)
        del self._row[name]
        del self.hits[name]
        self._spare.append(row)
        self._spare.sort()

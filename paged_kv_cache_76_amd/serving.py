"""Iterated decode steps over a paged cache: the per-iteration work of a
serving engine restricted to the attention hot path.

Each step, for every running sequence, the host block manager appends one
slot (allocating a block when the last one is full, copying a shared partial
block first), the copies run as one batched ``pa_copy_blocks``, the new
tokens' keys/values are written by ``pa_reshape_and_cache`` and
``pa_paged_decode`` attends over the whole history.  Finished sequences give
their blocks back.

Sources: "vLLM / PagedAttention" (awesome.papernotes.org), key designs 2-3
(on-demand allocation, reference counts, copy-on-write) and 5 (fused write,
attention and batched copy kernels); "vLLM" notes (formulaic.cloudchewie.com),
"在不同解码策略下的效果" (parallel sampling shares the prompt's blocks; beam
search forks candidates from surviving parents and releases pruned ones);
"vLLM / PagedAttention (SOSP 2023)" guide, section 03 (finished requests
release their blocks).

The new tokens' q/k/v are seeded N(0,1) draws standing in for a model's
projections (no weights are available).  Host histories of every running
sequence are kept (as lists of per-step chunks, shared between forked
sequences) so a checker can rebuild any sequence's logical history.
"""

from __future__ import annotations

import math
import time
from dataclasses import dataclass, field

import numpy as np
import torch

from . import inputs
from ._lib import (KVCache, decode_grouped_workspace, decode_workspace, pa_copy_blocks, pa_paged_decode,
                   pa_paged_decode_append, pa_paged_decode_grouped, pa_reshape_and_cache)
from .block_manager import BlockManager
from .workloads import STREAMS, TORCH


@dataclass
class StepRecord:
    rows: np.ndarray           # batch rows decoded this step (ascending)
    context_lens: np.ndarray   # their context lengths (new token included)
    n_copies: int
    out: torch.Tensor          # device [len(rows)][H][d]
    q: torch.Tensor            # host queries of this step
    gpu_ms: float | None = None


@dataclass
class History:
    """A sequence's logical K/V history as a list of host chunks [n][H][d]."""

    k: list = field(default_factory=list)
    v: list = field(default_factory=list)

    def fork(self) -> "History":
        return History(list(self.k), list(self.v))

    def materialise(self):
        return torch.cat(self.k), torch.cat(self.v)


class ServingLoop:
    """A batch of sequences decoding one token per step.

    ``prompt_lens[s]`` tokens of prompt plus ``start[s]`` already generated
    tokens are in the cache at step 0; sequence ``s`` finishes after
    ``out_lens[s]`` generated tokens (its blocks are freed then).
    ``fused``: each step's new tokens are written by the decode launch itself
    (pa_paged_decode_append) instead of a pa_reshape_and_cache launch before it.
    """

    def __init__(self, config_index: int, prompt_lens, out_lens, start, num_heads: int, head_dim: int,
                 block_size: int, dtype: str, device: str = "cuda", keep_history: bool = True,
                 slack: float = 1.10, out_dtype: torch.dtype | None = None, fused: bool = False):
        prompt_lens = np.asarray(prompt_lens, np.int64)
        self.out_lens = np.asarray(out_lens, np.int64)
        start = np.asarray(start, np.int64)
        self.S = len(prompt_lens)
        self.H, self.d, self.B = num_heads, head_dim, block_size
        self.dtype, self.device = dtype, device
        self.fused = fused
        self.out_dtype = out_dtype or TORCH[dtype]
        self.scale = 1.0 / math.sqrt(head_dim)
        self.generated = start.copy()
        lens0 = prompt_lens + start
        self.total_lens = prompt_lens + self.out_lens
        _, _, r_k, r_v, r_pool, r_step, _ = inputs.streams(config_index, STREAMS)
        self.r_step = r_step
        # every block the batch will ever hold, plus head-room
        need = int(sum(-(-int(L) // block_size) for L in self.total_lens))
        N = int(math.ceil(need * slack))
        self.max_blocks = -(-int(self.total_lens.max()) // block_size)
        self.mgr = BlockManager(N, block_size, max_rows=self.S, max_blocks_per_seq=self.max_blocks,
                                free_order=inputs.pool_order(r_pool, N))
        self.cache = KVCache.empty(N + 1, num_heads, block_size, head_dim, TORCH[dtype], device)
        self.cache.k.fill_(float("nan"))
        self.cache.v.fill_(float("nan"))
        total = int(lens0.sum())
        k_all = inputs.normal(r_k, (total, num_heads, head_dim), dtype)
        v_all = inputs.normal(r_v, (total, num_heads, head_dim), dtype)
        cuts = np.concatenate([[0], np.cumsum(lens0)])
        slots = np.concatenate([self.mgr.add_prompt(s, int(lens0[s])) for s in range(self.S)])
        pa_reshape_and_cache(self.cache, k_all.to(device), v_all.to(device), torch.from_numpy(slots).to(device))
        self.keep_history = keep_history
        self.hist = [History([k_all[cuts[s]:cuts[s + 1]]], [v_all[cuts[s]:cuts[s + 1]]]) if keep_history
                     else None for s in range(self.S)]
        # sized for the whole batch at its longest: every later step fits
        self.ws = decode_workspace(self.cache, self.S, int(self.total_lens.max()))
        self.bm_seconds = 0.0  # host time spent in the block manager

    # ---- one step -------------------------------------------------------------
    def active_rows(self) -> np.ndarray:
        return np.nonzero((self.generated < self.out_lens) & (self.mgr.lens[: self.S] > 0))[0]

    def active_counts(self, steps: int) -> list[int]:
        """Rows running at each of the next ``steps`` steps (deterministic)."""
        return [int(np.count_nonzero(self.generated + t < self.out_lens)) for t in range(steps)]

    def tokens(self, n: int, device: str | None = None):
        """The next step's synthetic activations for ``n`` rows: seeded
        N(0,1) (k, v, q), standing in for a model's projections."""
        k = inputs.normal(self.r_step, (n, self.H, self.d), self.dtype)
        v = inputs.normal(self.r_step, (n, self.H, self.d), self.dtype)
        q = inputs.normal(self.r_step, (n, self.H, self.d), self.dtype)
        if device is not None:
            k, v, q = k.to(device), v.to(device), q.to(device)
        return k, v, q

    def plan(self, rows: np.ndarray):
        """Host half of a step: the block manager's append for ``rows`` and the
        integer inputs the kernels need, staged in pinned memory."""
        t0 = time.perf_counter()
        slots, pairs = self.mgr.append_step(rows)
        tables = np.ascontiguousarray(self.mgr.tables[rows])
        lens = self.mgr.lens[rows].astype(np.int32)
        self.bm_seconds += time.perf_counter() - t0
        host = {"slots": torch.from_numpy(slots), "pairs": torch.from_numpy(pairs),
                "tables": torch.from_numpy(tables), "lens": torch.from_numpy(lens)}
        if self.device != "cpu" and torch.cuda.is_available():
            host = {k: t.pin_memory() for k, t in host.items()}
        return host, lens

    def launch(self, rows: np.ndarray, host: dict, lens: np.ndarray, toks, events=None) -> StepRecord:
        """Device half of a step: upload the plan, copy-on-write copies, write,
        decode.  ``toks`` = (k, v, q) for the rows, on the device."""
        dev = {k: t.to(self.device, non_blocking=True) for k, t in host.items()}
        k_new, v_new, q = toks
        max_ctx = int(lens.max())
        out = torch.empty((len(rows), self.H, self.d), dtype=self.out_dtype, device=self.device)
        if events is not None:
            events[0].record()
        if host["pairs"].shape[0]:
            pa_copy_blocks(self.cache, dev["pairs"])
        if self.fused:
            # rows ascend, as in append_step: each row's new token is the newest of its table row
            pa_paged_decode_append(self.cache, out, q, k_new, v_new, dev["tables"], dev["lens"], max_ctx,
                                   self.scale, 1, self.ws)
        else:
            pa_reshape_and_cache(self.cache, k_new, v_new, dev["slots"])
            pa_paged_decode(self.cache, out, q, dev["tables"], dev["lens"], max_ctx, self.scale, self.ws)
        if events is not None:
            events[1].record()
        return StepRecord(rows, lens, int(host["pairs"].shape[0]), out, None)

    def finish(self, rows: np.ndarray, toks_host=None) -> None:
        """Bookkeeping after a step: histories, progress, freeing."""
        if self.keep_history and toks_host is not None:
            k, v, _ = toks_host
            for i, s in enumerate(rows):
                self.hist[s].k.append(k[i:i + 1])
                self.hist[s].v.append(v[i:i + 1])
        t0 = time.perf_counter()
        self.generated[rows] += 1
        for s in rows:
            if self.generated[s] >= self.out_lens[s]:
                self.mgr.free(int(s))
        self.bm_seconds += time.perf_counter() - t0

    def step(self, events=None, toks=None) -> StepRecord | None:
        """One whole step.  Without ``toks`` the activations are drawn on the
        host (and kept for the histories); with ``toks`` (device tensors for
        the running rows) nothing but the plan crosses to the device."""
        rows = self.active_rows()
        if len(rows) == 0:
            return None
        host, lens = self.plan(rows)
        toks_host = None
        if toks is None:
            toks_host = self.tokens(len(rows))
            toks = tuple(t.to(self.device) for t in toks_host)
        rec = self.launch(rows, host, lens, toks, events)
        if toks_host is not None:
            rec.q = toks_host[2]
        self.finish(rows, toks_host)
        return rec


def opt13b_serving_lengths(config_index: int = 3, S: int = 256):
    """Prompt / output / progress draws of the serving-loop workload: prompts
    lognormal (median 160, sigma 1) in [1, 1024]; outputs lognormal (median
    300, sigma 1) >= 1, prompt + output <= 2048; each sequence is caught at a
    uniform point of its output (a steady-state snapshot of iteration-level
    serving)."""
    r_len = inputs.streams(config_index, STREAMS)[0]
    prompt = inputs.lognormal_lengths(r_len, S, 160, 1.0, 1, 1024)
    out = inputs.lognormal_lengths(r_len, S, 300, 1.0, 1, None)
    out = np.minimum(out, 2048 - prompt)
    start = np.floor(inputs.uniform_fraction(r_len, S) * out).astype(np.int64)
    return prompt, out, start


class BeamLoop:
    """Groups of ``width`` sequences sharing a prompt: parallel sampling
    (children never re-parent) or beam search (every step each group's
    children fork from parents drawn with replacement, then the previous
    generation is released).  Rows alternate between two halves of the
    table so a generation can fork into the other half.  ``fused``: as for
    ServingLoop (the decode launch writes the step's new tokens)."""

    def __init__(self, config_index: int, groups: int, width: int, prompt_len: int, steps: int,
                 num_heads: int, head_dim: int, block_size: int, dtype: str, beam: bool,
                 device: str = "cuda", keep_history: bool = True, slack: float = 1.25, grouped: bool = False,
                 fused: bool = False):
        self.G, self.W, self.beam = groups, width, beam
        self.fused = fused
        # fused steps also fold their copy-on-write copies into the decode launch
        self.fold_copies = fused
        self.copy_launches = 0  # pa_copy_blocks launches made by the steps
        self.H, self.d, self.B = num_heads, head_dim, block_size
        self.dtype, self.device = dtype, device
        self.scale = 1.0 / math.sqrt(head_dim)
        n = groups * width
        _, _, r_k, r_v, r_pool, r_step, r_beam = inputs.streams(config_index, STREAMS)
        self.r_step, self.r_beam = r_step, r_beam
        prompt_blocks = -(-prompt_len // block_size)
        grow = -(-steps // block_size) + 2
        # shared prompt blocks once per group + per-sequence growth (x2 while forking)
        N = int(math.ceil((groups * prompt_blocks + 2 * n * grow) * slack))
        self.max_blocks = prompt_blocks + grow
        self.mgr = BlockManager(N, block_size, max_rows=2 * n, max_blocks_per_seq=self.max_blocks,
                                free_order=inputs.pool_order(r_pool, N))
        self.cache = KVCache.empty(N + 1, num_heads, block_size, head_dim, TORCH[dtype], device)
        self.cache.k.fill_(float("nan"))
        self.cache.v.fill_(float("nan"))
        k_all = inputs.normal(r_k, (groups * prompt_len, num_heads, head_dim), dtype)
        v_all = inputs.normal(r_v, (groups * prompt_len, num_heads, head_dim), dtype)
        slots = []
        self.keep_history = keep_history
        self.hist = {}
        for gi in range(groups):
            root = gi * width
            slots.append(self.mgr.add_prompt(root, prompt_len))
            for c in range(1, width):
                self.mgr.fork(root, root + c)     # the prompt's blocks, reference count = width
            if keep_history:
                kh = k_all[gi * prompt_len:(gi + 1) * prompt_len]
                vh = v_all[gi * prompt_len:(gi + 1) * prompt_len]
                for c in range(width):
                    self.hist[root + c] = History([kh], [vh])
        pa_reshape_and_cache(self.cache, k_all.to(device), v_all.to(device),
                             torch.from_numpy(np.concatenate(slots)).to(device))
        self.cur = np.arange(n)
        self.nxt = np.arange(n, 2 * n)
        # grouped: the decode batch's rows come group by group, so the width
        # sequences sharing a prompt form one group of pa_paged_decode_grouped
        self.grouped = grouped
        if grouped:
            self.ws = decode_grouped_workspace(self.cache, n, prompt_len + steps + 1, width)
        else:
            self.ws = decode_workspace(self.cache, n, prompt_len + steps + 1)

    def remap(self) -> None:
        """Beam search: the children of each group fork from parents drawn
        with replacement (sorted); the previous generation is released."""
        parents = inputs.choice_with_replacement(self.r_beam, self.G, self.W)
        for gi in range(self.G):
            for c in range(self.W):
                src = int(self.cur[gi * self.W + parents[gi, c]])
                dst = int(self.nxt[gi * self.W + c])
                self.mgr.fork(src, dst)
                if self.keep_history:
                    self.hist[dst] = self.hist[src].fork()
        for s in self.cur:
            self.mgr.free(int(s))
            if self.keep_history:
                del self.hist[int(s)]
        self.cur, self.nxt = self.nxt, self.cur

    def plan(self) -> dict:
        """Host half of a step: the beam-search remap, the block manager's
        append (slots and copy-on-write pairs), the new tokens' activations,
        the history bookkeeping, and the upload of everything the kernels read.
        Plans can be made ahead of their launches: the kernels' effect on the
        pools depends only on the order in which the plans are launched."""
        if self.beam:
            self.remap()
        rows = self.cur
        slots, pairs = self.mgr.append_step(rows)
        order = np.argsort(rows, kind="stable")   # append_step reports rows ascending
        rows_sorted = rows[order]
        n = len(rows)
        k_new = inputs.normal(self.r_step, (n, self.H, self.d), self.dtype)
        v_new = inputs.normal(self.r_step, (n, self.H, self.d), self.dtype)
        q = inputs.normal(self.r_step, (n, self.H, self.d), self.dtype)
        lens = self.mgr.lens[rows_sorted].astype(np.int32)
        tables = np.ascontiguousarray(self.mgr.tables[rows_sorted])
        copy_pairs, cow = pairs, None
        newest = tables[np.arange(n), (lens - 1) // self.B]
        # tokens the copies carry: each copy's destination is the newest-token
        # block of the row that appends into it, which holds (len - 1) % B
        # of that row's tokens before the newest
        cow_tokens = 0
        for _, dst in pairs:
            hit = np.nonzero(newest == dst)[0]
            cow_tokens += int(lens[hit[0]] - 1) % self.B if len(hit) else self.B
        if self.fold_copies:
            # that row takes the copy's source instead
            cow = np.full(n, -1, np.int32)
            left = []
            for src, dst in pairs:
                hit = np.nonzero(newest == dst)[0]
                if len(hit) == 1:
                    cow[hit[0]] = src
                else:
                    left.append((src, dst))
            copy_pairs = np.asarray(left, np.int64).reshape(-1, 2)
        dev = {"pairs": torch.from_numpy(copy_pairs), "k": k_new, "v": v_new, "slots": torch.from_numpy(slots),
               "q": q, "tables": torch.from_numpy(tables), "lens": torch.from_numpy(lens)}
        if cow is not None:
            dev["cow"] = torch.from_numpy(cow)
        dev = {k: t.to(self.device) for k, t in dev.items()}
        if self.keep_history:
            for i, s in enumerate(rows_sorted):
                self.hist[int(s)].k.append(k_new[i:i + 1])
                self.hist[int(s)].v.append(v_new[i:i + 1])
        return {"rows": rows_sorted, "lens": lens, "n_pairs": len(pairs), "cow_tokens": cow_tokens,
                "n_copy_launch": len(copy_pairs),
                "dev": dev, "q": q, "max_ctx": int(lens.max())}

    def launch(self, plan: dict, events=None) -> StepRecord:
        """Device half of a step: copy-on-write copies, the new tokens' cache
        write and the decode, bracketed by ``events`` if given."""
        dev = plan["dev"]
        n = len(plan["rows"])
        out = torch.empty((n, self.H, self.d), dtype=TORCH[self.dtype], device=self.device)
        if events is not None:
            events[0].record()
        if plan["n_copy_launch"]:
            pa_copy_blocks(self.cache, dev["pairs"])
            self.copy_launches += 1
        if self.fused:
            pa_paged_decode_append(self.cache, out, dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"],
                                   plan["max_ctx"], self.scale, self.W if self.grouped else 1, self.ws,
                                   cow_src=dev.get("cow"))
        else:
            self._write_and_decode(plan, out)
        if events is not None:
            events[1].record()
        return StepRecord(plan["rows"], plan["lens"], plan["n_pairs"], out, plan["q"])

    def _write_and_decode(self, plan: dict, out: torch.Tensor) -> None:
        dev = plan["dev"]
        pa_reshape_and_cache(self.cache, dev["k"], dev["v"], dev["slots"])
        if self.grouped:
            pa_paged_decode_grouped(self.cache, out, dev["q"], dev["tables"], dev["lens"], plan["max_ctx"],
                                    self.scale, self.W, self.ws)
        else:
            pa_paged_decode(self.cache, out, dev["q"], dev["tables"], dev["lens"], plan["max_ctx"], self.scale,
                            self.ws)

    def step(self, events=None) -> StepRecord:
        return self.launch(self.plan(), events)

    def decode_only(self, plan: dict) -> torch.Tensor:
        """The decode launch of ``plan`` alone, for timing it again after the
        steps have run.  It leaves the cache as it is: the plain decode only
        reads, and a fused loop's appending decode stores each row's newest
        token again, with the bits already there."""
        dev = plan["dev"]
        out = torch.empty((len(plan["rows"]), self.H, self.d), dtype=TORCH[self.dtype], device=self.device)
        if self.fused:
            pa_paged_decode_append(self.cache, out, dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"],
                                   plan["max_ctx"], self.scale, self.W if self.grouped else 1, self.ws)
        elif self.grouped:
            pa_paged_decode_grouped(self.cache, out, dev["q"], dev["tables"], dev["lens"], plan["max_ctx"],
                                    self.scale, self.W, self.ws)
        else:
            pa_paged_decode(self.cache, out, dev["q"], dev["tables"], dev["lens"], plan["max_ctx"], self.scale,
                            self.ws)
        return out

    def warm(self, plan: dict) -> None:
        """Launch this loop's kernels once, leaving the cache as the timed
        steps expect it: a copy of block 0 onto itself and the decode of
        ``plan``'s inputs (read-only; for a fused loop the appending decode
        stores ``plan``'s new tokens early, into blocks no row reads yet, and
        ``plan``'s own launch stores them again after its copies).  The first
        launch of each kernel in a process loads its code, which must not
        fall inside timed steps."""
        dev = plan["dev"]
        out = torch.empty((len(plan["rows"]), self.H, self.d), dtype=TORCH[self.dtype], device=self.device)
        pa_copy_blocks(self.cache, torch.zeros((1, 2), dtype=torch.int64, device=self.device))
        if self.fused:
            pa_paged_decode_append(self.cache, out, dev["q"], dev["k"], dev["v"], dev["tables"], dev["lens"],
                                   plan["max_ctx"], self.scale, self.W if self.grouped else 1, self.ws)
        elif self.grouped:
            pa_paged_decode_grouped(self.cache, out, dev["q"], dev["tables"], dev["lens"], plan["max_ctx"],
                                    self.scale, self.W, self.ws)
        else:
            pa_paged_decode(self.cache, out, dev["q"], dev["tables"], dev["lens"], plan["max_ctx"], self.scale,
                            self.ws)

    def unique_blocks_read(self, rows) -> int:
        """Distinct physical blocks the decode of ``rows`` reads."""
        ids = set()
        for s in rows:
            ids.update(self.mgr.table(int(s)))
        return len(ids)

"""Synthetic paged-decode workloads at the pages' shapes, built through the
host block manager and the C-ABI (the K/V histories are written into the
pools by ``pa_reshape_and_cache``).

The pages measure on OPT models (OPT-13B: 40 heads of 128, 2-byte KV) with
ShareGPT/Alpaca length mixes that are not available here; these seeded
generators stand in for them (see :mod:`paged_kv_cache_76_amd.inputs`).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

from . import inputs
from ._lib import KVCache, pa_copy_blocks, pa_reshape_and_cache
from .block_manager import BlockManager, PrefixCache

TORCH = inputs.DTYPES

# children of a workload's seed: 0 lengths, 1 queries, 2 keys, 3 values,
# 4 pool order, 5 decode-step tokens, 6 beam choices
STREAMS = 7


@dataclass
class DecodeBatch:
    """One layer's paged cache plus one decode step's inputs, resident on the
    device, with the host copies the checkers read."""

    cache: KVCache
    manager: BlockManager
    q: torch.Tensor            # host [S][H][d], storage dtype
    k_hist: list               # host per sequence [L_s][H][d]
    v_hist: list
    q_dev: torch.Tensor
    tables_dev: torch.Tensor   # int32 [S][max_blocks]
    lens_dev: torch.Tensor     # int32 [S]
    lens: np.ndarray
    max_context_len: int
    scale: float

    @property
    def S(self) -> int:
        return self.q.shape[0]


def pool_blocks(lens, block_size: int, slack: float = 1.10, extra: int = 0) -> int:
    """Physical blocks for the histories plus ``slack`` head-room (and
    ``extra`` blocks for later growth)."""
    need = int(sum(-(-int(L) // block_size) for L in lens))
    return max(1, int(math.ceil(need * slack)) + extra)


@dataclass
class HostHistories:
    """The host half of a decode batch: histories, queries, block manager and
    the slots the histories go to."""

    manager: BlockManager
    q: torch.Tensor
    k_all: torch.Tensor        # [sum L][H][d], sequences back to back
    v_all: torch.Tensor
    k_hist: list
    v_hist: list
    slots: np.ndarray          # int64 [sum L]
    lens: np.ndarray


def host_histories(config_index: int, lens, num_heads: int, head_dim: int, block_size: int,
                   dtype: str, slack: float = 1.10, extra_blocks: int = 0,
                   grow_tokens: int = 0) -> HostHistories:
    """Seeded histories of ``lens[s]`` tokens, placed by the block manager
    into a seeded-shuffled pool of ``pool_blocks(lens) + extra_blocks``."""
    lens = np.asarray(lens, dtype=np.int64)
    S = len(lens)
    _, r_q, r_k, r_v, r_pool = inputs.streams(config_index, STREAMS)[:5]
    N = pool_blocks(lens, block_size, slack, extra_blocks)
    max_blocks = -(-(int(lens.max()) + grow_tokens) // block_size)
    mgr = BlockManager(N, block_size, max_rows=S, max_blocks_per_seq=max_blocks,
                       free_order=inputs.pool_order(r_pool, N))
    total = int(lens.sum())
    k_all = inputs.normal(r_k, (total, num_heads, head_dim), dtype)
    v_all = inputs.normal(r_v, (total, num_heads, head_dim), dtype)
    q = inputs.normal(r_q, (S, num_heads, head_dim), dtype)
    cuts = np.concatenate([[0], np.cumsum(lens)])
    k_hist = [k_all[cuts[s]:cuts[s + 1]] for s in range(S)]
    v_hist = [v_all[cuts[s]:cuts[s + 1]] for s in range(S)]
    slots = np.concatenate([mgr.add_prompt(s, int(lens[s])) for s in range(S)])
    return HostHistories(mgr, q, k_all, v_all, k_hist, v_hist, slots, lens)


def build_decode_batch(config_index: int, lens, num_heads: int, head_dim: int, block_size: int,
                       dtype: str, device: str = "cuda", slack: float = 1.10, extra_blocks: int = 0,
                       grow_tokens: int = 0, nan_fill: bool = True) -> DecodeBatch:
    """Histories of ``lens[s]`` tokens each (the last one is the token being
    decoded), written through seeded-shuffled blocks, plus one query per
    sequence.

    The device pool has one block more than the manager owns: that block (id
    ``num_blocks``, the table's poison id) and every slot never written are
    filled with NaN, so a read of anything outside a sequence's history shows
    up in the output.
    """
    h = host_histories(config_index, lens, num_heads, head_dim, block_size, dtype, slack,
                       extra_blocks, grow_tokens)
    mgr = h.manager
    cache = KVCache.empty(mgr.num_blocks + 1, num_heads, block_size, head_dim, TORCH[dtype], device)
    if nan_fill:
        cache.k.fill_(float("nan"))
        cache.v.fill_(float("nan"))
    pa_reshape_and_cache(cache, h.k_all.to(device), h.v_all.to(device),
                         torch.from_numpy(h.slots).to(device))
    return DecodeBatch(
        cache=cache, manager=mgr, q=h.q, k_hist=h.k_hist, v_hist=h.v_hist, q_dev=h.q.to(device),
        tables_dev=torch.from_numpy(mgr.tables).to(device),
        lens_dev=torch.from_numpy(h.lens.astype(np.int32)).to(device),
        lens=h.lens, max_context_len=int(h.lens.max()), scale=1.0 / math.sqrt(head_dim))


def opt13b_decode_lengths(config_index: int = 2, S: int = 64, lo: int = 1, hi: int = 2048) -> np.ndarray:
    """Context lengths of the OPT-13B decode workload: uniform on [1, 2048]."""
    r_len = inputs.streams(config_index, STREAMS)[0]
    return inputs.uniform_lengths(r_len, S, lo, hi)


def decode_bytes(lens, num_heads: int, head_dim: int, elem_bytes: int, block_size: int) -> int:
    """Algorithmic HBM bytes of one decode launch: every valid K and V row
    once, q and out once, and the table entries in use."""
    lens = np.asarray(lens, dtype=np.int64)
    S = len(lens)
    kv = int(lens.sum()) * 2 * num_heads * head_dim * elem_bytes
    qo = 2 * S * num_heads * head_dim * elem_bytes
    tbl = 4 * int(sum(-(-int(L) // block_size) for L in lens))
    return kv + qo + tbl + 4 * S


@dataclass
class PrefillBatch:
    """Prompts whose K/V sit in the paged cache, plus the query rows of the
    last ``q_lens[s]`` positions of each, resident on the device."""

    cache: KVCache
    manager: BlockManager
    q: torch.Tensor            # host [sum q][H][d]
    k_hist: list
    v_hist: list
    q_dev: torch.Tensor
    tables_dev: torch.Tensor
    cu_q_dev: torch.Tensor     # int32 [S+1]
    lens_dev: torch.Tensor
    lens: np.ndarray
    q_lens: np.ndarray
    cu_q: np.ndarray
    scale: float


def build_prefill_batch(config_index: int, lens, q_lens, num_heads: int, head_dim: int, block_size: int,
                        dtype: str, device: str = "cuda", slack: float = 1.10,
                        nan_fill: bool = True) -> PrefillBatch:
    """Histories of ``lens[s]`` tokens written through seeded-shuffled blocks
    (as :func:`build_decode_batch`), and seeded queries for the last
    ``q_lens[s]`` positions of every sequence."""
    lens = np.asarray(lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    if q_lens.shape != lens.shape or np.any(q_lens < 1) or np.any(q_lens > lens):
        raise ValueError("need 1 <= q_lens[s] <= lens[s]")
    h = host_histories(config_index, lens, num_heads, head_dim, block_size, dtype, slack)
    r_step = inputs.streams(config_index, STREAMS)[5]
    q = inputs.normal(r_step, (int(q_lens.sum()), num_heads, head_dim), dtype)
    mgr = h.manager
    cache = KVCache.empty(mgr.num_blocks + 1, num_heads, block_size, head_dim, TORCH[dtype], device)
    if nan_fill:
        cache.k.fill_(float("nan"))
        cache.v.fill_(float("nan"))
    pa_reshape_and_cache(cache, h.k_all.to(device), h.v_all.to(device), torch.from_numpy(h.slots).to(device))
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return PrefillBatch(
        cache=cache, manager=mgr, q=q, k_hist=h.k_hist, v_hist=h.v_hist, q_dev=q.to(device),
        tables_dev=torch.from_numpy(mgr.tables).to(device), cu_q_dev=torch.from_numpy(cu_q).to(device),
        lens_dev=torch.from_numpy(lens.astype(np.int32)).to(device), lens=lens, q_lens=q_lens, cu_q=cu_q,
        scale=1.0 / math.sqrt(head_dim))


def prefill_flops(lens, q_lens, num_heads: int, head_dim: int) -> int:
    """Algorithmic flops of causal prefill: 2 matmuls x 2 flops x d for every
    (query, key <= query) pair."""
    total = 0
    for L, n in zip(np.asarray(lens, np.int64), np.asarray(q_lens, np.int64)):
        first = int(L - n)
        # query positions first .. L-1 attend to first+1 .. L keys
        total += (n * (first + 1) + n * (n - 1) // 2)
    return 4 * head_dim * num_heads * int(total)


def prefill_bytes(lens, q_lens, num_heads: int, head_dim: int, elem_bytes: int, block_size: int) -> int:
    """Algorithmic HBM bytes of one prefill launch: every query row read and
    every output row written once, every key and value row of the contexts
    read once, the table entries in use, the query offsets and the lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    q_lens = np.asarray(q_lens, dtype=np.int64)
    row = num_heads * head_dim * elem_bytes
    qo = 2 * int(q_lens.sum()) * row
    kv = 2 * int(lens.sum()) * row
    tbl = 4 * int(sum(-(-int(L) // block_size) for L in lens))
    return qo + kv + tbl + 4 * (2 * len(lens) + 1)


@dataclass
class LongDecode:
    """Long-context decode: histories generated on the device by a seeded
    torch generator (no host copy of the 19 GB), written through the block
    manager's slots; host copies are kept only for the sampled (sequence,
    head) pairs a checker asks for."""

    cache: KVCache
    manager: BlockManager
    q_dev: torch.Tensor
    tables_dev: torch.Tensor
    lens_dev: torch.Tensor
    lens: np.ndarray
    scale: float
    samples: dict              # (seq, head) -> (q [d], K [L][d], V [L][d]) host tensors


def build_long_decode(config_index: int, S: int, ctx: int, num_heads: int, head_dim: int, block_size: int,
                      dtype: str, samples=(), slack: float = 1.02, chunk_tokens: int = 8192) -> LongDecode:
    """``S`` sequences of ``ctx`` tokens each, N(0,1) keys/values/queries drawn
    on the device from ``torch.Generator`` seeded with 76000 + config_index."""
    lens = np.full(S, ctx, dtype=np.int64)
    r_pool = inputs.streams(config_index, STREAMS)[4]
    N = pool_blocks(lens, block_size, slack)
    mgr = BlockManager(N, block_size, max_rows=S, max_blocks_per_seq=-(-ctx // block_size),
                       free_order=inputs.pool_order(r_pool, N))
    cache = KVCache.empty(N + 1, num_heads, block_size, head_dim, TORCH[dtype], "cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(76_000 + config_index)
    want = {}
    for s, h in samples:
        want.setdefault(s, []).append(h)
    kept = {}
    for s in range(S):
        slots = torch.from_numpy(mgr.add_prompt(s, ctx)).cuda()
        ks, vs = [], []
        for t0 in range(0, ctx, chunk_tokens):
            n = min(chunk_tokens, ctx - t0)
            k = torch.randn((n, num_heads, head_dim), generator=gen, device="cuda").to(TORCH[dtype])
            v = torch.randn((n, num_heads, head_dim), generator=gen, device="cuda").to(TORCH[dtype])
            pa_reshape_and_cache(cache, k, v, slots[t0:t0 + n])
            if s in want:
                ks.append(k[:, want[s]].cpu())
                vs.append(v[:, want[s]].cpu())
        if s in want:
            kept[s] = (torch.cat(ks), torch.cat(vs))
    q = torch.randn((S, num_heads, head_dim), generator=gen, device="cuda").to(TORCH[dtype])
    sample_data = {}
    for s, heads in want.items():
        K, V = kept[s]
        for i, h in enumerate(heads):
            sample_data[(s, h)] = (q[s, h].cpu(), K[:, i], V[:, i])
    return LongDecode(cache, mgr, q, torch.from_numpy(mgr.tables).cuda(),
                      torch.from_numpy(lens.astype(np.int32)).cuda(), lens, 1.0 / math.sqrt(head_dim), sample_data)


@dataclass
class PrefixBatch:
    """Requests that map a provider's cached prefix and prefill only their
    own task input ("vLLM / PagedAttention (SOSP 2023)" guide, section 04)."""

    cache: KVCache
    manager: BlockManager
    prefix_k: torch.Tensor     # host [P][H][d]
    prefix_v: torch.Tensor
    task_k: list               # host per request [T_i][H][d]
    task_v: list
    q: torch.Tensor            # host [sum T_i][H][d], queries of the task tokens
    q_dev: torch.Tensor
    tables_dev: torch.Tensor   # int32 [R][max_blocks] (rows 1..R of the manager)
    cu_q_dev: torch.Tensor
    lens_dev: torch.Tensor
    lens: np.ndarray           # prefix + task
    task_lens: np.ndarray
    cu_q: np.ndarray
    copies: int
    scale: float


def build_shared_prefix(config_index: int, prefix_len: int, task_lens, num_heads: int, head_dim: int,
                        block_size: int, dtype: str, device: str = "cuda") -> PrefixBatch:
    """Row 0 of the block manager holds a provider prefix of ``prefix_len``
    tokens (written once); request i forks it, extends by ``task_lens[i]``
    tokens (copying the partial last prefix block first) and writes its own
    keys/values.  Queries cover the task tokens only."""
    task_lens = np.asarray(task_lens, np.int64)
    R = len(task_lens)
    _, r_q, r_k, r_v, r_pool, _, _ = inputs.streams(config_index, STREAMS)
    max_len = prefix_len + int(task_lens.max())
    need = -(-prefix_len // block_size) + int(sum(-(-(int(t) + block_size) // block_size) for t in task_lens))
    N = int(math.ceil(need * 1.1)) + 1
    mgr = BlockManager(N, block_size, max_rows=R + 1, max_blocks_per_seq=-(-max_len // block_size),
                       free_order=inputs.pool_order(r_pool, N))
    cache = KVCache.empty(N + 1, num_heads, block_size, head_dim, TORCH[dtype], device)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    pk = inputs.normal(r_k, (prefix_len, num_heads, head_dim), dtype)
    pv = inputs.normal(r_v, (prefix_len, num_heads, head_dim), dtype)
    pslots = mgr.add_prompt(0, prefix_len)
    pa_reshape_and_cache(cache, pk.to(device), pv.to(device), torch.from_numpy(pslots).to(device))
    tk, tv, all_slots, all_pairs = [], [], [], []
    for i, t in enumerate(task_lens, start=1):
        mgr.fork(0, i)
        slots, pairs = mgr.extend(i, int(t))
        all_slots.append(slots)
        all_pairs.append(pairs)
        tk.append(inputs.normal(r_k, (int(t), num_heads, head_dim), dtype))
        tv.append(inputs.normal(r_v, (int(t), num_heads, head_dim), dtype))
    pairs = np.concatenate(all_pairs) if all_pairs else np.zeros((0, 2), np.int64)
    if len(pairs):  # copy-on-write of the shared partial block, before any task write
        pa_copy_blocks(cache, torch.from_numpy(pairs).to(device))
    pa_reshape_and_cache(cache, torch.cat(tk).to(device), torch.cat(tv).to(device),
                         torch.from_numpy(np.concatenate(all_slots)).to(device))
    q = inputs.normal(r_q, (int(task_lens.sum()), num_heads, head_dim), dtype)
    lens = (prefix_len + task_lens).astype(np.int64)
    cu_q = np.concatenate([[0], np.cumsum(task_lens)]).astype(np.int32)
    return PrefixBatch(cache, mgr, pk, pv, tk, tv, q, q.to(device),
                       torch.from_numpy(np.ascontiguousarray(mgr.tables[1:R + 1])).to(device),
                       torch.from_numpy(cu_q).to(device), torch.from_numpy(lens.astype(np.int32)).to(device),
                       lens, task_lens, cu_q, len(pairs), 1.0 / math.sqrt(head_dim))


@dataclass
class PrefixSetBatch:
    """Requests over a provider's set of cached prefixes, each prefilling only
    its own task input ("vLLM / PagedAttention (SOSP 2023)" guide, section 04)."""

    cache: KVCache
    manager: BlockManager
    prefixes: PrefixCache
    prefix_k: dict             # name -> host [P][H][d]
    prefix_v: dict
    request_prefix: list       # prefix name of each request
    task_k: list               # host per request [T_i][H][d]
    task_v: list
    q: torch.Tensor            # host [sum T_i][H][d]
    q_dev: torch.Tensor
    tables_dev: torch.Tensor   # int32 [R][max_blocks] (request rows)
    cu_q_dev: torch.Tensor
    lens_dev: torch.Tensor
    lens: np.ndarray
    task_lens: np.ndarray
    cu_q: np.ndarray
    copies: int
    scale: float


def build_prefix_set(config_index: int, prefix_lens: dict, requests, num_heads: int, head_dim: int,
                     block_size: int, dtype: str, device: str = "cuda") -> PrefixSetBatch:
    """Register the provider prefixes ``prefix_lens`` (name -> tokens) in a
    PrefixCache and write their keys/values; then each request ``(name,
    task_len)`` attaches its prefix, copies a shared partial last block if its
    first task token lands there, and writes its own task keys/values.
    Queries cover the task tokens only."""
    R = len(requests)
    _, r_q, r_k, r_v, r_pool, _, _ = inputs.streams(config_index, STREAMS)
    names = sorted(prefix_lens)
    max_len = max(prefix_lens[n] + t for n, t in requests)
    need = sum(-(-int(prefix_lens[n]) // block_size) for n in names) + \
        int(sum(-(-(int(t) + block_size) // block_size) for _, t in requests))
    N = int(math.ceil(need * 1.1)) + 1
    mgr = BlockManager(N, block_size, max_rows=R + len(names), max_blocks_per_seq=-(-max_len // block_size),
                       free_order=inputs.pool_order(r_pool, N))
    pc = PrefixCache(mgr, rows=range(R, R + len(names)))
    cache = KVCache.empty(N + 1, num_heads, block_size, head_dim, TORCH[dtype], device)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    pk, pv = {}, {}
    for n in names:
        pk[n] = inputs.normal(r_k, (prefix_lens[n], num_heads, head_dim), dtype)
        pv[n] = inputs.normal(r_v, (prefix_lens[n], num_heads, head_dim), dtype)
        slots = pc.register(n, prefix_lens[n])
        pa_reshape_and_cache(cache, pk[n].to(device), pv[n].to(device), torch.from_numpy(slots).to(device))
    tk, tv, all_slots, all_pairs = [], [], [], []
    for i, (n, t) in enumerate(requests):
        slots, pairs = pc.attach(n, i, int(t))
        all_slots.append(slots)
        all_pairs.append(pairs)
        tk.append(inputs.normal(r_k, (int(t), num_heads, head_dim), dtype))
        tv.append(inputs.normal(r_v, (int(t), num_heads, head_dim), dtype))
    pairs = np.concatenate(all_pairs) if all_pairs else np.zeros((0, 2), np.int64)
    if len(pairs):  # copy-on-write of shared partial prefix blocks, before any task write
        pa_copy_blocks(cache, torch.from_numpy(pairs).to(device))
    pa_reshape_and_cache(cache, torch.cat(tk).to(device), torch.cat(tv).to(device),
                         torch.from_numpy(np.concatenate(all_slots)).to(device))
    task_lens = np.array([int(t) for _, t in requests], np.int64)
    q = inputs.normal(r_q, (int(task_lens.sum()), num_heads, head_dim), dtype)
    lens = np.array([prefix_lens[n] + int(t) for n, t in requests], np.int64)
    cu_q = np.concatenate([[0], np.cumsum(task_lens)]).astype(np.int32)
    return PrefixSetBatch(cache, mgr, pc, pk, pv, [n for n, _ in requests], tk, tv, q, q.to(device),
                          torch.from_numpy(np.ascontiguousarray(mgr.tables[:R])).to(device),
                          torch.from_numpy(cu_q).to(device), torch.from_numpy(lens.astype(np.int32)).to(device),
                          lens, task_lens, cu_q, len(pairs), 1.0 / math.sqrt(head_dim))

"""What a slot-mapped cache write and a batched block copy leave in the pools.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: "vLLM / PagedAttention" (awesome.papernotes.org), key design 5
(new keys/values are reshaped into the block-read layout and written into
their slots; copy-on-write triggers block copies that are batched into one
operation), key design 3 (copy-on-write copies the old block's content into
the new block); "vLLM" notes (formulaic.cloudchewie.com), "PagedAttention
原理" (the prompt's K/V are written into the physical-block slots that the
block table maps to).

Readings taken where the pages are silent:

* Pool layout: separate key and value pools, each ``[num_blocks][H][B][d]``;
  token offset ``o`` of head ``h`` in physical block ``b`` lives at
  ``pool[b, h, o, :]``.
* Slot encoding: ``slot = b * B + o`` as a signed 64-bit integer; a negative
  slot means "do not write this token".
* A copy moves the whole block — every slot, every head, keys and values.

Both functions return new arrays and leave their inputs untouched, so a test
can compare every byte of the expected pool with the device pool.
"""

from __future__ import annotations

import numpy as np


def reshape_and_cache(k_pool: np.ndarray, v_pool: np.ndarray,
                      key: np.ndarray, value: np.ndarray,
                      slot_mapping) -> tuple[np.ndarray, np.ndarray]:
    """Expected pools after writing ``key, value [T][H][d]`` into their slots.

    For each token ``t`` with ``slot_mapping[t] >= 0``:
    ``pool[slot // B, :, slot % B, :] = kv[t]``.  Slots are unique within a
    call (a precondition of the write), so the order of tokens is immaterial.
    """
    if k_pool.shape != v_pool.shape or key.shape != value.shape:
        raise ValueError("pool or token shapes differ between K and V")
    N, H, B, d = k_pool.shape
    T = key.shape[0]
    if key.shape != (T, H, d):
        raise ValueError(f"token rows {key.shape} do not match pool {k_pool.shape}")
    slots = [int(s) for s in np.asarray(slot_mapping).reshape(-1)]
    if len(slots) != T:
        raise ValueError("one slot per token is required")
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        block, offset = divmod(slot, B)
        if block >= N:
            raise IndexError(f"slot {slot} is outside a pool of {N} blocks")
        k_out[block, :, offset, :] = key[t]
        v_out[block, :, offset, :] = value[t]
    return k_out, v_out


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray,
                pairs) -> tuple[np.ndarray, np.ndarray]:
    """Expected pools after copying whole blocks ``dst <- src`` for each pair.

    ``pairs`` is a sequence of ``(src, dst)`` physical ids.  Destinations are
    distinct and no destination is also a source (a precondition of the
    batched copy), so every copy reads the pool as it was before the call.
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_out[dst] = k_pool[src]
        v_out[dst] = v_pool[src]
    return k_out, v_out


def swap_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                pairs) -> tuple[np.ndarray, np.ndarray]:
    """Expected destination pools after copying whole blocks from one pool to
    another (device <-> host swapping, "vLLM" notes, 调度和抢占): for each
    ``(src, dst)``, ``dst_pool[dst] = src_pool[src]`` for keys and values."""
    k_out = dst_k.copy()
    v_out = dst_v.copy()
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_out[dst] = src_k[src]
        v_out[dst] = src_v[src]
    return k_out, v_out


def gather_history(pool: np.ndarray, block_table, context_len: int) -> np.ndarray:
    """The logically contiguous ``[L][H][d]`` history of one sequence, read
    through its block table: logical position ``p`` is slot ``p % B`` of
    physical block ``table[p // B]`` ("vLLM" notes, "PagedAttention 原理":
    the block table translates logical blocks to physical ones)."""
    N, H, B, d = pool.shape
    out = np.empty((context_len, H, d), dtype=pool.dtype)
    for p in range(context_len):
        out[p] = pool[int(block_table[p // B]), :, p % B, :]
    return out

"""Pins of the cache-write and block-copy oracle.

The write is pinned by an independent vectorised formulation (the pool seen
as ``[N*B][H][d]`` slot rows) and by read-back through block tables built by
the block model; the copy by whole-block equality, order independence and
untouched-bytes checks.

Sources: "vLLM / PagedAttention" (awesome.papernotes.org), key design 5 (fused
reshape and block write; batched block copy) and key design 3
(copy-on-write); "vLLM" notes (formulaic.cloudchewie.com), "PagedAttention
原理" (prompt K/V written into the slots the block table maps to).
"""

import numpy as np
import pytest

from oracle import block_model as bm
from oracle import cache as oc


def _pools(r, N, H, B, d):
    return r.standard_normal((N, H, B, d)).astype(np.float32), r.standard_normal((N, H, B, d)).astype(np.float32)


def _slot_rows(pool):
    # independent view: slot s = b*B + o  <->  row s of [N*B][H][d]
    N, H, B, d = pool.shape
    return pool.transpose(0, 2, 1, 3).reshape(N * B, H, d)


def test_write_equals_slot_row_scatter():
    r = np.random.default_rng(0)
    N, H, B, d, T = 10, 3, 4, 8, 17
    kp, vp = _pools(r, N, H, B, d)
    key = r.standard_normal((T, H, d)).astype(np.float32)
    val = r.standard_normal((T, H, d)).astype(np.float32)
    slots = r.choice(N * B, size=T, replace=False).astype(np.int64)
    slots[[2, 9]] = -1                            # skipped tokens
    k2, v2 = oc.reshape_and_cache(kp, vp, key, val, slots)
    ek, ev = _slot_rows(kp).copy(), _slot_rows(vp).copy()
    keep = slots >= 0
    ek[slots[keep]] = key[keep]
    ev[slots[keep]] = val[keep]
    assert np.array_equal(_slot_rows(k2), ek)
    assert np.array_equal(_slot_rows(v2), ev)
    # inputs untouched
    assert not np.shares_memory(k2, kp)


def test_write_then_gather_through_table_reconstructs_history():
    r = np.random.default_rng(1)
    N, H, B, d = 32, 2, 4, 8
    model = bm.BlockModel(N, B, r.permutation(N))
    kp, vp = _pools(r, N, H, B, d)
    hist = {}
    for sid, L in enumerate([7, 1, 12, 4]):
        slots = model.add_prompt(sid, L)
        k = r.standard_normal((L, H, d)).astype(np.float32)
        kp, vp = oc.reshape_and_cache(kp, vp, k, -k, slots)
        hist[sid] = k
    for step in range(6):                          # decode steps, lazy append
        for sid in sorted(hist):
            slot, pair = model.append(sid)
            assert pair is None
            k = r.standard_normal((1, H, d)).astype(np.float32)
            kp, vp = oc.reshape_and_cache(kp, vp, k, -k, [slot])
            hist[sid] = np.concatenate([hist[sid], k])
    for sid, k in hist.items():
        L = model.length(sid)
        assert np.array_equal(oc.gather_history(kp, model.table(sid), L), k)
        assert np.array_equal(oc.gather_history(vp, model.table(sid), L), -k)


def test_write_rejects_out_of_pool_slot():
    r = np.random.default_rng(2)
    kp, vp = _pools(r, 2, 1, 4, 8)
    kv = np.zeros((1, 1, 8), np.float32)
    with pytest.raises(IndexError):
        oc.reshape_and_cache(kp, vp, kv, kv, [8])


def test_copy_moves_whole_blocks_and_nothing_else():
    r = np.random.default_rng(3)
    N, H, B, d = 12, 3, 4, 8
    kp, vp = _pools(r, N, H, B, d)
    pairs = [(1, 5), (1, 7), (9, 0), (4, 11)]
    k2, v2 = oc.copy_blocks(kp, vp, pairs)
    dsts = {dst for _, dst in pairs}
    for src, dst in pairs:
        assert np.array_equal(k2[dst], kp[src]) and np.array_equal(v2[dst], vp[src])
    for b in range(N):
        if b not in dsts:
            assert np.array_equal(k2[b], kp[b]) and np.array_equal(v2[b], vp[b])
    # the order of pairs does not matter under the precondition
    k3, v3 = oc.copy_blocks(kp, vp, pairs[::-1])
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3)


def test_copy_on_write_keeps_both_histories():
    # parallel sampling: two samples share a partial block; the first writer copies
    r = np.random.default_rng(4)
    N, H, B, d = 8, 1, 4, 8
    model = bm.BlockModel(N, B, r.permutation(N))
    kp, vp = _pools(r, N, H, B, d)
    prompt = r.standard_normal((7, H, d)).astype(np.float32)
    kp, vp = oc.reshape_and_cache(kp, vp, prompt, prompt, model.add_prompt(0, 7))
    model.fork(0, 1)
    new = {}
    for sid in (0, 1):
        slot, pair = model.append(sid)
        if pair is not None:
            kp, vp = oc.copy_blocks(kp, vp, [pair])
        new[sid] = r.standard_normal((1, H, d)).astype(np.float32)
        kp, vp = oc.reshape_and_cache(kp, vp, new[sid], new[sid], [slot])
    for sid in (0, 1):
        expect = np.concatenate([prompt, new[sid]])
        assert np.array_equal(oc.gather_history(kp, model.table(sid), 8), expect)


def test_swap_blocks_copies_across_pools():
    r = np.random.default_rng(5)
    dk, dv = _pools(r, 6, 2, 4, 8)
    hk, hv = _pools(r, 4, 2, 4, 8)
    pairs = [(5, 0), (1, 3)]
    k2, v2 = oc.swap_blocks(dk, dv, hk, hv, pairs)
    assert np.array_equal(k2[0], dk[5]) and np.array_equal(v2[3], dv[1])
    assert np.array_equal(k2[1], hk[1]) and np.array_equal(k2[2], hk[2])
    # and back: a round trip restores the device pool bit for bit
    dk2, dv2 = oc.swap_blocks(k2, v2, np.zeros_like(dk), np.zeros_like(dv), [(0, 5), (3, 1)])
    assert np.array_equal(dk2[5], dk[5]) and np.array_equal(dv2[1], dv[1])

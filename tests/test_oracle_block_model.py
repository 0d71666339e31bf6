"""Pins of the block-manager model: the pages' two worked examples, the
beam-search release walk, the tail-waste and physical-count identities, and
brute-force enumeration of short operation sequences with a data-level check
that every sequence still reads back its own history.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import block_model as bm

from conftest import GOLDEN


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _order_with_prefix(prefix, n):
    rest = [i for i in range(n) if i not in prefix]
    return list(prefix) + rest


def test_worked_example_single_request():
    g = _golden("worked_example_single_request.json")
    B = g["block_size"]
    m = bm.BlockModel(16, B, _order_with_prefix(g["free_order_prefix"], 16))
    m.add_prompt(0, g["prompt_len"])
    assert len(m.table(0)) == g["after_prefill"]["table_len"]
    assert m.filled(0) == g["after_prefill"]["filled"]
    assert m.table(0)[0] == g["after_prefill"]["first_physical"]
    for step in (1, 2, 3):
        slot, pair = m.append(0)
        assert pair is None
        want = g[f"after_decode_{step}"]
        assert len(m.table(0)) == want["table_len"]
        assert m.filled(0) == want["filled"]
        m.check_invariants()
    # the first decoded token landed in the reserved slot of logical block 1
    assert m.slot(0, 7) == m.table(0)[1] * B + 3


def test_worked_example_parallel_sampling_copy_on_write():
    g = _golden("worked_example_parallel_sampling.json")
    B = g["block_size"]
    m = bm.BlockModel(8, B, _order_with_prefix(g["free_order_prefix"], 8))
    m.add_prompt(1, g["prompt_len"])       # A1
    m.fork(1, 2)                           # A2 shares the prompt blocks
    a = g["after_prefill"]
    assert m.table(1) == a["A1"] and m.table(2) == a["A2"]
    assert {str(k): v for k, v in m.ref.items()} == a["ref"]
    _, pair1 = m.append(1)                 # A1 writes first and copies
    _, pair2 = m.append(2)                 # A2 writes in place
    d = g["after_decode_1"]
    assert m.table(1) == d["A1"] and m.table(2) == d["A2"]
    assert {str(k): v for k, v in m.ref.items()} == d["ref"]
    assert [list(p) for p in m.copies] == d["copies"]
    assert pair1 == (1, 3) and pair2 is None
    m.check_invariants()


def test_full_and_shared_last_block_gets_a_new_block_without_copy():
    m = bm.BlockModel(8, 4, list(range(8)))
    m.add_prompt(0, 8)                     # two full blocks
    m.fork(0, 1)
    s0, p0 = m.append(0)
    s1, p1 = m.append(1)
    assert p0 is None and p1 is None
    assert m.table(0)[:2] == m.table(1)[:2] and m.table(0)[2] != m.table(1)[2]
    m.check_invariants()


def test_beam_search_prunes_back_to_the_shared_root():
    # "vLLM" notes, Beam Search: candidates fork from surviving parents; pruned
    # candidates' blocks are released, walking back until the prompt block that
    # every candidate shares.
    B = 4
    m = bm.BlockModel(64, B, list(range(64)))
    m.add_prompt(0, 4)                     # the prompt block (full)
    for c in (1, 2, 3):
        m.fork(0, c)
    live = [0, 1, 2, 3]
    r = np.random.default_rng(0)
    next_id = 4
    for step in range(9):
        parents = sorted(r.integers(0, 4, size=4))
        children = []
        for p in parents:
            m.fork(live[p], next_id)
            children.append(next_id)
            next_id += 1
        for s in live:
            m.free(s)
        live = children
        for s in live:
            m.append(s)
        m.check_invariants()
    # the prompt block is shared by every live candidate; nothing else is held
    root = m.table(live[0])[0]
    assert all(m.table(s)[0] == root for s in live)
    assert m.ref[root] == 4
    held = set().union(*[set(m.table(s)) for s in live])
    assert set(m.ref) == held
    for s in live:
        m.free(s)
    assert m.used() == 0 and len(m.free_list) == 64


def test_out_of_blocks_and_double_free():
    m = bm.BlockModel(2, 4, [0, 1])
    m.add_prompt(0, 8)
    with pytest.raises(bm.OutOfBlocks):
        m.append(0)
    with pytest.raises(bm.OutOfBlocks):
        m.add_prompt(1, 1)
    m.free(0)
    with pytest.raises(KeyError):
        m.free(0)
    assert m.used() == 0


def test_tail_waste_bound_over_lengths():
    # key design 2, eq. 3: 0 <= waste < B slots (lazy allocation)
    for B in (1, 2, 4, 16):
        m = bm.BlockModel(4096, B, None)
        for L in range(1, 70):
            m.add_prompt(L, L)
            assert 0 <= m.tail_waste(L) <= B - 1
        m.check_invariants()


OPS = ("prompt1", "promptB1", "append", "fork", "free")


def _apply(model, data, op, rng_vals, next_sid):
    """One operation on the model and on a plain per-sequence list of token
    values (``data``); the pool content is tracked slot by slot in
    ``data['pool']`` so copy pairs and writes can be checked."""
    live = sorted(s for s in model.seqs)
    pool = data["pool"]
    if op in ("prompt1", "promptB1"):
        L = 1 if op == "prompt1" else model.B + 1
        try:
            slots = model.add_prompt(next_sid, L)
        except bm.OutOfBlocks:
            return next_sid
        vals = [next(rng_vals) for _ in range(L)]
        for s, v in zip(slots, vals):
            pool[s] = v
        data[next_sid] = vals
        return next_sid + 1
    if not live:
        return next_sid
    sid = live[0] if op != "append" else live[-1]
    if op == "append":
        try:
            slot, pair = model.append(sid)
        except bm.OutOfBlocks:
            return next_sid
        if pair is not None:
            src, dst = pair
            for o in range(model.B):
                if src * model.B + o in pool:
                    pool[dst * model.B + o] = pool[src * model.B + o]
        v = next(rng_vals)
        pool[slot] = v
        data[sid] = data[sid] + [v]
    elif op == "fork":
        model.fork(sid, next_sid)
        data[next_sid] = list(data[sid])
        return next_sid + 1
    elif op == "free":
        model.free(sid)
        del data[sid]
    return next_sid


@pytest.mark.parametrize("B", [1, 2, 4])
def test_brute_force_operation_sequences(B):
    # every sequence of 5 operations on a pool of 8 blocks: invariants hold and
    # each live sequence reads its own values back through its block table
    count = 0
    for ops in itertools.product(OPS, repeat=5):
        model = bm.BlockModel(8, B, [3, 6, 0, 7, 1, 4, 2, 5])
        data = {"pool": {}}
        vals = itertools.count(1)
        sid = 0
        for op in ops:
            sid = _apply(model, data, op, vals, sid)
            model.check_invariants()
            for s in model.seqs:
                got = [data["pool"][model.slot(s, p)] for p in range(model.length(s))]
                assert got == data[s], (ops, s)
        count += 1
    assert count == len(OPS) ** 5

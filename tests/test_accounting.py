"""KV-memory accounting of contiguous reservation vs paged blocks (host only)."""

import numpy as np

from paged_kv_cache_76_amd import accounting
from paged_kv_cache_76_amd.serving import opt13b_serving_lengths


def test_reserved_slots_by_hand():
    prompt, out, cur = np.array([10, 3]), np.array([5, 40]), np.array([12, 20])
    assert accounting.reserved_slots("max", prompt, out, cur, max_len=64).tolist() == [64, 64]
    assert accounting.reserved_slots("pow2", prompt, out, cur, max_len=64).tolist() == [10 + 8, 3 + 64 - 3]
    assert accounting.reserved_slots("oracle", prompt, out, cur).tolist() == [15, 43]
    assert accounting.reserved_slots("paged", prompt, out, cur, block_size=8).tolist() == [16, 24]


def test_paged_waste_is_below_one_block_per_request():
    # key design 2, eq. 3: held - used < B for every request
    r = np.random.default_rng(0)
    cur = r.integers(1, 3000, size=500)
    for B in (1, 8, 16, 32):
        held = accounting.reserved_slots("paged", cur, cur, cur, block_size=B)
        assert np.all((held - cur >= 0) & (held - cur < B))


def test_serving_length_mix_orders_the_policies():
    prompt, out, start = opt13b_serving_lengths()
    u = accounting.utilisation(prompt, out, prompt + start)
    assert u["max"] < u["pow2"] < u["oracle"] < u["paged"]
    assert u["paged"] > 0.95
    assert u["max"] < 0.3

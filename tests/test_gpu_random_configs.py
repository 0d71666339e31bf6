"""Seeded random configurations against the float64 oracle: the decode, the
appending decode (group 1, 2 or 4) and the prefill over every built
(dtype, head_dim, block_size), with the batch size, head count, context
lengths and query lengths drawn per case.  Lengths mix block, partition and
query-tile boundaries with uniform draws.  Every case is fixed by its index
(numpy's seeded generator) and prints its parameters before it runs.

What each must equal: [P1] key design 1, eq. 1 (softmax-weighted sum over the
positions up to the query's own, scale 1/sqrt(d)), computed by the oracle over
the logically contiguous histories; the appending decode's pools must also
equal the oracle's cache write bit for bit, and with copy-on-write folded in
the oracle's copy then write ([P1] key design 3: a write into a shared block
first copies it to a fresh block)."""

import numpy as np
import pytest
import torch

from oracle import cache as oc
from paged_kv_cache_76_amd import _lib as L
from paged_kv_cache_76_amd import workloads
from paged_kv_cache_76_amd.workloads import TORCH

from gpu_util import TOL, bits, check_close, from_bits, random_bits
from test_gpu_append import _run_case, cow_case
from test_gpu_decode import _oracle as _decode_oracle
from test_gpu_decode import _run as _decode_run
from test_gpu_prefill import _oracle as _prefill_oracle
from test_gpu_prefill import _run as _prefill_run
from test_gpu_swap import _pinned_from_bits

pytestmark = pytest.mark.gpu

DTYPES = ["f32", "f16", "bf16"]
# (head_dim, block_size) pairs the decode is built for
DECODE_SHAPES = [(8, 4), (8, 8), (8, 16), (64, 16), (64, 32), (128, 8), (128, 16), (128, 32), (128, 64),
                 (128, 128), (256, 16), (256, 32)]


def _lengths(rng, S, B, hi):
    """S context lengths in [1, hi]: about half from the boundaries of a
    block, a narrow partition (1024) and a wide one (4096), the rest uniform."""
    special = np.array([1, 2, B - 1, B, B + 1, 2 * B + 1, 1023, 1024, 1025, 4095, 4096, 4097])
    special = special[(special >= 1) & (special <= hi)]
    uniform = rng.integers(1, hi + 1, S)
    pick = rng.random(S) < 0.5
    return [int(x) for x in np.where(pick, rng.choice(special, S), uniform)]


def _decode_case(i):
    rng = np.random.default_rng(7690 + i)
    dtype = DTYPES[i % 3]
    d, B = DECODE_SHAPES[(i // 3 + i) % len(DECODE_SHAPES)]
    if i % 4 == 3:
        # 32 rows x 32 heads of short contexts: the wide partitioning
        d = min(d, 128)
        return dtype, d, B, 32, 32, _lengths(rng, 32, B, 200)
    S = int(rng.integers(1, 9))
    H = int(rng.integers(1, 7))
    return dtype, d, B, S, H, _lengths(rng, S, B, 5000)


@pytest.mark.parametrize("i", range(48))
def test_random_decode(i):
    dtype, d, B, S, H, lens = _decode_case(i)
    print(f"random decode {i}: {dtype} d={d} B={B} S={S} H={H} lens={lens}", flush=True)
    b = workloads.build_decode_batch(8000 + i, lens, num_heads=H, head_dim=d, block_size=B, dtype=dtype)
    check_close(_decode_run(b), _decode_oracle(b), TOL[dtype], f"random decode {i}")


@pytest.mark.parametrize("i", range(36))
def test_random_appending_decode(i):
    rng = np.random.default_rng(7790 + i)
    dtype = DTYPES[i % 3]
    if i % 2 == 0:
        # the grouped builds: head_dim 128, blocks of 16 or 32, groups of 2 or 4
        d, B, group = 128, (16, 32)[(i // 2) % 2], (2, 4)[(i // 4) % 2]
    else:
        d, B = DECODE_SHAPES[(i * 5) % len(DECODE_SHAPES)]
        group = 1
    S = int(rng.integers(1, 11))
    H = int(rng.integers(1, 6))
    lens = _lengths(rng, S, B, 4500)
    print(f"random appending decode {i}: {dtype} d={d} B={B} group={group} S={S} H={H} lens={lens}", flush=True)
    _run_case(8100 + i, lens, H, d, B, dtype, group=group)


@pytest.mark.parametrize("i", range(36))
def test_random_prefill(i):
    rng = np.random.default_rng(7890 + i)
    if i % 2 == 0:
        # the MFMA kernel: head_dim 128, bf16 or f16, blocks of 16 to 128
        dtype, d, B = ("bf16", "f16")[(i // 2) % 2], 128, (16, 32, 64, 128)[(i // 2) % 4]
    else:
        # the generic kernel: any other description
        dtype = DTYPES[(i // 2) % 3]
        d, B = ((8, 4), (64, 16), (256, 32), (128, 16), (32, 8), (96, 2))[(i // 2) % 6]
        if d == 128 and dtype != "f32":
            dtype = "f32"
    S = int(rng.integers(1, 5))
    H = int(rng.integers(1, 5))
    special = np.array([1, 2, B - 1, B, B + 1, 63, 64, 65, 127, 128, 129, 255, 257, 640])
    special = special[special >= 1]
    lens = [int(x) for x in np.where(rng.random(S) < 0.5, rng.choice(special, S), rng.integers(1, 700, S))]
    # the queries: the whole prompt, or its last q_len positions
    q_lens = [int(n) if rng.random() < 0.5 else int(rng.integers(1, n + 1)) for n in lens]
    print(f"random prefill {i}: {dtype} d={d} B={B} S={S} H={H} lens={lens} q_lens={q_lens}", flush=True)
    b = workloads.build_prefill_batch(8200 + i, lens, q_lens, num_heads=H, head_dim=d, block_size=B, dtype=dtype)
    out = _prefill_run(b).cpu()
    for s in range(S):
        check_close(out[b.cu_q[s]:b.cu_q[s + 1]], _prefill_oracle(b, s), TOL[dtype], f"random prefill {i} seq {s}")


@pytest.mark.parametrize("i", range(24))
def test_random_copy_on_write_in_the_appending_decode(i):
    # prompts forked into 2-4 rows each; the first append after the fork
    # writes into the shared partial last block, so all rows but the last
    # sharer copy it (cow_src) and the appending decode does copies, writes
    # and decode in one launch
    rng = np.random.default_rng(7990 + i)
    dtype = DTYPES[i % 3]
    d = 64 if i % 4 == 0 else 128
    B = (16, 32)[(i // 4) % 2] if d == 64 else (8, 16, 32, 64, 128)[(i // 3) % 5]
    W = (1, 2, 4)[(i // 2) % 3]
    width = int(rng.integers(2, 5))
    groups = int(rng.integers(1, 5))
    H = int(rng.integers(1, 6))
    kind = i % 3
    if kind == 0:      # anywhere, at any offset within the last block
        prompt = int(rng.integers(1, 1200 // B)) * B + int(rng.integers(1, B))
    elif kind == 1:    # the copied block one token short of full
        prompt = int(rng.integers(1, 1200 // B)) * B + B - 1
    else:              # the copied block just past the first narrow partition
        prompt = 1024 + int(rng.integers(1, B))
    print(f"random copy-on-write {i}: {dtype} d={d} B={B} W={W} width={width} groups={groups} H={H} "
          f"prompt={prompt}", flush=True)
    cow_case(8300 + i, W, dtype, B, prompt, [1] * width, H=H, d=d, groups=groups)


# ---- the byte operations: any cache description (rows of a multiple of 16
# bytes, power-of-two blocks), bit-exact over every byte of the pools, which
# start as random bits ([P1] key designs 3 and 5: whole-block copies, batched;
# [P2] "PagedAttention 原理": each token's K/V go to the slot its table maps)

def _pools(i, base):
    rng = np.random.default_rng(base + i)
    dtype = DTYPES[i % 3]
    t = TORCH[dtype]
    d = (8, 16, 64, 96, 128, 256)[int(rng.integers(0, 6))]
    B = (1, 2, 4, 8, 16, 32, 64, 128)[int(rng.integers(0, 8))]
    H = int(rng.integers(1, 9))
    N = int(rng.integers(2, 48))
    return rng, dtype, t, N, H, B, d


@pytest.mark.parametrize("i", range(24))
def test_random_reshape_and_cache(i):
    rng, dtype, t, N, H, B, d = _pools(i, 8400)
    T = int(rng.integers(1, N * B + 1))
    slots = rng.choice(N * B, size=T, replace=False).astype(np.int64)
    slots[rng.random(T) < 0.1] = -1                      # skipped tokens
    print(f"random write {i}: {dtype} N={N} H={H} B={B} d={d} T={T}", flush=True)
    kb, vb = random_bits(rng, (N, H, B, d), t), random_bits(rng, (N, H, B, d), t)
    keyb, valb = random_bits(rng, (T, H, d), t), random_bits(rng, (T, H, d), t)
    cache = L.KVCache(from_bits(kb, t), from_bits(vb, t))
    L.pa_reshape_and_cache(cache, from_bits(keyb, t), from_bits(valb, t), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    ek, ev = oc.reshape_and_cache(kb, vb, keyb, valb, slots)
    assert np.array_equal(bits(cache.k), ek) and np.array_equal(bits(cache.v), ev)


def _pairs(rng, n_src, n_dst, n, same_pool):
    """n (src, dst) pairs with distinct destinations; in one pool no
    destination is also a source (sources may repeat)."""
    dst = rng.choice(n_dst, size=n, replace=False)
    pool = np.setdiff1d(np.arange(n_src), dst) if same_pool else np.arange(n_src)
    src = rng.choice(pool, size=n, replace=True)
    return np.stack([src, dst], axis=1).astype(np.int64)


@pytest.mark.parametrize("i", range(24))
def test_random_copy_blocks(i):
    rng, dtype, t, N, H, B, d = _pools(i, 8500)
    n = int(rng.integers(1, N // 2 + 1))
    pairs = _pairs(rng, N, N, n, same_pool=True)
    print(f"random copy {i}: {dtype} N={N} H={H} B={B} d={d} pairs={n}", flush=True)
    kb, vb = random_bits(rng, (N, H, B, d), t), random_bits(rng, (N, H, B, d), t)
    cache = L.KVCache(from_bits(kb, t), from_bits(vb, t))
    L.check_copy_pairs(pairs, N, N)
    L.pa_copy_blocks(cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    ek, ev = oc.copy_blocks(kb, vb, pairs)
    assert np.array_equal(bits(cache.k), ek) and np.array_equal(bits(cache.v), ev)


@pytest.mark.parametrize("dma", [False, True])
@pytest.mark.parametrize("i", range(12))
def test_random_swap_round_trip(i, dma):
    # out to a host pool (its own size), then back in to other device blocks;
    # the copy-engine form with a staging buffer of a drawn number of blocks
    rng, dtype, t, N, H, B, d = _pools(i, 8600 + (100 if dma else 0))
    NH = int(rng.integers(1, N + 1))
    n = int(rng.integers(1, min(N, NH) + 1))
    out_pairs = _pairs(rng, N, NH, n, same_pool=False)
    in_pairs = np.stack([out_pairs[:, 1], rng.choice(N, size=n, replace=False)], axis=1).astype(np.int64)
    stage_blocks = int(rng.integers(1, n + 1))
    print(f"random swap {i} dma={dma}: {dtype} N={N} NH={NH} H={H} B={B} d={d} pairs={n} staging={stage_blocks}",
          flush=True)
    dk, dv = random_bits(rng, (N, H, B, d), t), random_bits(rng, (N, H, B, d), t)
    hk, hv = random_bits(rng, (NH, H, B, d), t), random_bits(rng, (NH, H, B, d), t)
    cache = L.KVCache(from_bits(dk, t), from_bits(dv, t))
    host_k, host_v = _pinned_from_bits(hk, t), _pinned_from_bits(hv, t)
    staging = L.swap_staging(cache, stage_blocks) if dma else None

    def swap(pairs, direction):
        if dma:
            L.pa_swap_blocks_dma(cache, host_k, host_v, pairs, direction, staging)
        else:
            L.pa_swap_blocks(cache, host_k, host_v, torch.from_numpy(pairs).cuda(), direction)
        torch.cuda.synchronize()

    swap(out_pairs, L.PA_SWAP_OUT)
    ek, ev = oc.swap_blocks(dk, dv, hk, hv, out_pairs)
    assert np.array_equal(bits(host_k), ek) and np.array_equal(bits(host_v), ev)
    assert np.array_equal(bits(cache.k), dk) and np.array_equal(bits(cache.v), dv)   # sources untouched
    swap(in_pairs, L.PA_SWAP_IN)
    fk, fv = oc.swap_blocks(ek, ev, dk, dv, in_pairs)
    assert np.array_equal(bits(cache.k), fk) and np.array_equal(bits(cache.v), fv)

"""The C-ABI library loads, exports every symbol ``include/pagedattn.h``
declares, and rejects bad arguments on the host (no GPU is touched: every
call below fails validation before any HIP call, or is a documented no-op).
"""

import ctypes
import os
import re

import pytest
import torch

from paged_kv_cache_76_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libpagedattn.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert sorted(L.EXPORTS) == _declared()


def test_every_declared_symbol_is_exported():
    lib = L.lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = L.lib()
    assert lib.pa_abi_version() == 1
    assert lib.pa_status_string(L.PA_ERR_WORKSPACE) == b"PA_ERR_WORKSPACE"
    assert lib.pa_status_string(99) == b"PA_ERR_UNKNOWN"


FAKE = 0x10000  # aligned, never dereferenced: every call below stops on the host


def _desc(**kw):
    d = dict(k=FAKE, v=FAKE, num_blocks=8, num_heads=2, head_dim=128, block_size=16, dtype=L.PA_F16)
    d.update(kw)
    return L.PaKVCache(**d)


def _err(status, fragment):
    lib = L.lib()
    assert status != L.PA_OK
    assert fragment in lib.pa_last_error().decode(), lib.pa_last_error().decode()
    return status


@pytest.mark.parametrize("kw,code,frag", [
    (dict(block_size=3), L.PA_ERR_INVALID_ARG, "power of two"),
    (dict(block_size=0), L.PA_ERR_INVALID_ARG, ">= 1"),
    (dict(dtype=7), L.PA_ERR_INVALID_ARG, "dtype"),
    (dict(k=FAKE + 4), L.PA_ERR_INVALID_ARG, "aligned"),
    (dict(v=0), L.PA_ERR_INVALID_ARG, "NULL"),
    (dict(head_dim=4), L.PA_ERR_UNSUPPORTED, "multiple of 16"),
])
def test_cache_description_checks(kw, code, frag):
    d = _desc(**kw)
    st = L.lib().pa_copy_blocks(ctypes.byref(d), FAKE, 1, None)
    assert st == code
    _err(st, frag)


def test_null_cache_and_negative_sizes():
    lib = L.lib()
    assert lib.pa_copy_blocks(None, FAKE, 1, None) == L.PA_ERR_INVALID_ARG
    d = _desc()
    _err(lib.pa_copy_blocks(ctypes.byref(d), FAKE, -1, None), "< 0")
    _err(lib.pa_reshape_and_cache(ctypes.byref(d), FAKE, FAKE, FAKE, -2, None), "< 0")
    _err(lib.pa_reshape_and_cache(ctypes.byref(d), FAKE + 8, FAKE, FAKE, 4, None), "aligned")
    _err(lib.pa_reshape_and_cache(ctypes.byref(d), FAKE, FAKE, None, 4, None), "NULL")


def test_empty_calls_are_noops():
    lib = L.lib()
    d = _desc()
    assert lib.pa_copy_blocks(ctypes.byref(d), None, 0, None) == L.PA_OK
    assert lib.pa_reshape_and_cache(ctypes.byref(d), None, None, None, 0, None) == L.PA_OK
    assert lib.pa_paged_decode(ctypes.byref(d), None, L.PA_F16, None, None, 1, None, 0, 1, 1.0,
                               None, 0, None) == L.PA_OK


def test_decode_argument_checks():
    lib = L.lib()
    d = _desc()

    def call(out_dtype=L.PA_F16, maxb=8, maxctx=100, scale=0.1, ws=None, wsb=0, S=4):
        return lib.pa_paged_decode(ctypes.byref(d), FAKE, out_dtype, FAKE, FAKE, maxb, FAKE, S, maxctx,
                                   scale, ws, wsb, None)

    _err(call(out_dtype=L.PA_BF16), "out_dtype")
    _err(call(maxb=2), "cannot hold")
    _err(call(maxctx=0), "max_context_len")
    _err(call(scale=float("inf")), "scale")
    need = lib.pa_decode_workspace_bytes(ctypes.byref(d), 4, 6000)
    assert need > 0
    assert call(maxb=400, maxctx=6000, ws=FAKE, wsb=need - 1) == L.PA_ERR_WORKSPACE
    assert call(maxb=400, maxctx=6000, ws=None, wsb=need) == L.PA_ERR_WORKSPACE
    d2 = _desc(head_dim=48)
    assert lib.pa_paged_decode(ctypes.byref(d2), FAKE, L.PA_F16, FAKE, FAKE, 8, FAKE, 4, 100, 0.1, None, 0,
                               None) == L.PA_ERR_UNSUPPORTED


def test_append_decode_argument_checks():
    lib = L.lib()
    d = _desc()

    def call(key=FAKE, value=FAKE, group=1, maxctx=100, ws=None, wsb=0, S=4, maxb=8, cow=None, desc=d):
        return lib.pa_paged_decode_append(ctypes.byref(desc), FAKE, L.PA_F16, FAKE, key, value, cow, FAKE, maxb,
                                          FAKE, S, maxctx, 0.1, group, ws, wsb, None)

    _err(call(key=None), "NULL key/value")
    _err(call(value=FAKE + 8), "key/value must be 16-byte aligned")
    _err(call(cow=FAKE + 2), "cow_src must be 4-byte aligned")
    # a launch whose work-items (decode and writer workgroups) overflow the
    # 32-bit grid size is refused before anything runs
    _err(call(S=1 << 22), "does not fit")
    _err(call(group=3), "group_size = 3")
    _err(call(maxb=2), "cannot hold")
    assert call(S=0) == L.PA_OK
    for g in (1, 2, 4):
        need = lib.pa_decode_grouped_workspace_bytes(ctypes.byref(d), 4, 6000, g)
        assert need > 0
        assert call(group=g, maxb=400, maxctx=6000, ws=FAKE, wsb=need - 1) == L.PA_ERR_WORKSPACE


def test_workspace_size_formula():
    lib = L.lib()
    d = _desc(num_heads=40)
    # a context that fits one partition needs no workspace
    assert lib.pa_decode_workspace_bytes(ctypes.byref(d), 64, 16) == 0
    # layout: per-(sequence, head) counters padded to 256 bytes, then one
    # (d + 2)-float partial per (sequence, head, partition)
    def counters(S):
        return -(-(S * 40 * 4) // 256) * 256

    n1 = lib.pa_decode_workspace_bytes(ctypes.byref(d), 64, 8192)
    n2 = lib.pa_decode_workspace_bytes(ctypes.byref(d), 128, 8192)
    assert n1 > 0 and n2 - counters(128) == 2 * (n1 - counters(64))
    assert (n1 - counters(64)) % (64 * 40 * (128 + 2) * 4) == 0
    bad = _desc(head_dim=48)
    assert lib.pa_decode_workspace_bytes(ctypes.byref(bad), 4, 100) == ctypes.c_size_t(-1).value


def test_one_decode_workspace_serves_every_smaller_call():
    # the size never decreases in S or max_context_len, so a workspace sized
    # once for the largest batch serves every step of a shrinking batch
    lib = L.lib()
    for heads in (1, 8, 40, 72):
        d = _desc(num_heads=heads)
        Ss, Ls = [1, 2, 5, 16, 20, 64, 256], [1, 16, 1024, 1025, 2048, 4096, 4097, 32768]
        size = {(S, Lc): lib.pa_decode_workspace_bytes(ctypes.byref(d), S, Lc) for S in Ss for Lc in Ls}
        for (S, Lc), n in size.items():
            for (S2, L2), n2 in size.items():
                if S2 <= S and L2 <= Lc:
                    assert n2 <= n, (heads, S, Lc, S2, L2)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="no non-HIP fallback"):
        L.lib()


def test_prefill_argument_checks():
    lib = L.lib()
    d = _desc(dtype=L.PA_BF16)

    def call(out_dtype=L.PA_BF16, maxb=8, S=2, maxq=64, maxctx=100, scale=0.1):
        return lib.pa_paged_prefill(ctypes.byref(d), FAKE, out_dtype, FAKE, FAKE, maxb, FAKE, FAKE, S, maxq, maxctx,
                                    scale, None)

    _err(call(S=-1), "< 0")
    _err(call(out_dtype=L.PA_F16), "out_dtype")
    _err(call(maxq=0), "max_q_len")
    _err(call(maxq=101), "max_q_len")
    _err(call(maxb=2), "cannot hold")
    # the causal kernel orders raw scores by value, which needs a positive scale
    _err(call(scale=float("nan")), "scale")
    _err(call(scale=0.0), "> 0")
    _err(call(scale=-0.1), "> 0")
    # head dims beyond the generic kernel's 512 are not built
    d2 = _desc(dtype=L.PA_BF16, head_dim=1024)
    assert lib.pa_paged_prefill(ctypes.byref(d2), FAKE, L.PA_BF16, FAKE, FAKE, 8, FAKE, FAKE, 2, 64, 100, 0.1,
                                None) == L.PA_ERR_UNSUPPORTED
    # a grid beyond the 32-bit launch limits is refused, not truncated
    _err(call(S=1 << 20, maxq=1 << 14, maxctx=1 << 14, maxb=1 << 14), "launch limit")


def test_binding_refuses_host_tensors():
    # host pools (or any host tensor among device ones) must never reach a kernel
    cache = L.KVCache(torch.zeros((4, 2, 16, 128), dtype=torch.float16),
                      torch.zeros((4, 2, 16, 128), dtype=torch.float16))
    q = torch.zeros((2, 2, 128), dtype=torch.float16)
    tables = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="one GPU"):
        L.pa_paged_decode(cache, q.clone(), q, tables, lens, 1, 0.1)
    with pytest.raises(ValueError, match="one GPU"):
        L.pa_reshape_and_cache(cache, q, q.clone(), torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="one GPU"):
        L.pa_copy_blocks(cache, torch.zeros((1, 2), dtype=torch.int64))
    cu = torch.tensor([0, 1, 2], dtype=torch.int32)
    with pytest.raises(ValueError, match="one GPU"):
        L.pa_paged_prefill(cache, q.clone(), q, tables, cu, lens, 1, 1, 0.1)
    # a query whose head count differs from the pools' is refused by shape
    with pytest.raises(ValueError, match="query must be"):
        L.pa_paged_prefill(cache, q[:, :1].clone(), q[:, :1].clone(), tables, cu, lens, 1, 1, 0.1)


def test_binding_refuses_sizes_beyond_int32():
    # ctypes would wrap a size past int32 into another, smaller one (2**32 + 5
    # arrives as 5), so a call would silently cover part of the tensors: the
    # binding refuses such sizes before anything else sees them
    assert ctypes.CFUNCTYPE(ctypes.c_int32, ctypes.c_int32)(lambda x: x)((1 << 32) + 5) == 5
    with pytest.raises(ValueError, match="does not fit"):
        L._i32(T=(1 << 32) + 5)
    L._i32(T=(1 << 31) - 1, S=0, n=-(1 << 31))
    cache = L.KVCache(torch.zeros((4, 2, 16, 128), dtype=torch.float16),
                      torch.zeros((4, 2, 16, 128), dtype=torch.float16))
    q = torch.zeros((2, 2, 128), dtype=torch.float16)
    tables = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="max_context_len = 4294967297 does not fit"):
        L.pa_paged_decode(cache, q.clone(), q, tables, lens, (1 << 32) + 1, 0.1)
    cu = torch.tensor([0, 1, 2], dtype=torch.int32)
    with pytest.raises(ValueError, match="max_q_len = 4294967297 does not fit"):
        L.pa_paged_prefill(cache, q.clone(), q, tables, cu, lens, (1 << 32) + 1, (1 << 32) + 1, 0.1)
    with pytest.raises(ValueError, match="does not fit"):
        L.pa_decode_workspace_bytes(cache, 1 << 31, 16)


def test_read_helper_argument_checks():
    lib = L.lib()
    sink = ctypes.c_void_p(16)
    # sizes that are not multiples of 16, negative sizes, NULL and misaligned pointers
    assert lib.pa_read_stream(ctypes.c_void_p(4096), 24, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_stream(ctypes.c_void_p(4096), -16, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_stream(None, 32, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_stream(ctypes.c_void_p(4104), 32, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_stream(None, 0, None, None) == L.PA_OK  # no-op
    tiles = ctypes.c_void_p(64)
    assert lib.pa_read_tiles(ctypes.c_void_p(4096), 0, 4, tiles, 2, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_tiles(ctypes.c_void_p(4096), 40, 4, tiles, 2, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_tiles(ctypes.c_void_p(4096), 64, -1, tiles, 2, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_tiles(ctypes.c_void_p(4096), 64, 4, None, 2, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_tiles(ctypes.c_void_p(4096), 64, 4, ctypes.c_void_p(66), 2, sink, None) == L.PA_ERR_INVALID_ARG
    assert lib.pa_read_tiles(None, 64, 4, None, 0, None, None) == L.PA_OK  # no-op


def test_copy_swap_and_write_grids_beyond_the_launch_limit_are_refused():
    # 2n workgroups of 256 threads (copies, swaps) and T workgroups of 256
    # (writes) must fit the 32-bit work-item count of a launch dimension
    lib = L.lib()
    d = _desc()
    _err(lib.pa_copy_blocks(ctypes.byref(d), FAKE, 1 << 23, None), "launch limit")
    _err(lib.pa_swap_blocks(ctypes.byref(d), FAKE, FAKE, 8, FAKE, 1 << 23, L.PA_SWAP_OUT, None), "launch limit")
    _err(lib.pa_reshape_and_cache(ctypes.byref(d), FAKE, FAKE, FAKE, 1 << 24, None), "launch limit")


def test_swap_binding_refuses_mismatched_host_pools():
    # one host block count bounds both host pools in the kernel, so the
    # binding refuses host pools of different sizes before any launch
    cache = L.KVCache(torch.zeros((4, 2, 16, 128), dtype=torch.float16),
                      torch.zeros((4, 2, 16, 128), dtype=torch.float16))
    hk = torch.zeros((6, 2, 16, 128), dtype=torch.float16)
    hv = torch.zeros((3, 2, 16, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="same shape"):
        L.pa_swap_blocks(cache, hk, hv, torch.zeros((1, 2), dtype=torch.int64), L.PA_SWAP_OUT)


def test_swap_dma_argument_checks():
    # the copy-engine swap: bad arguments are refused before any HIP call
    lib = L.lib()
    d = _desc()
    pairs = (ctypes.c_int64 * 2)(0, 0)
    per_block = 2 * 2 * 16 * 128 * 2                        # a key and a value block of the description
    assert lib.pa_swap_staging_bytes(ctypes.byref(d), 3) == 3 * per_block
    assert lib.pa_swap_staging_bytes(ctypes.byref(d), 0) == 0

    def call(n=1, direction=L.PA_SWAP_OUT, hk=FAKE, dev_pairs=FAKE, staging=FAKE, nbytes=per_block):
        return lib.pa_swap_blocks_dma(ctypes.byref(d), hk, FAKE, 8, dev_pairs, pairs, n, direction, staging, nbytes,
                                      None)

    assert call(n=0) == L.PA_OK                               # no-op
    _err(call(direction=7), "bad direction")
    _err(call(n=-1), "negative size")
    _err(call(hk=None), "NULL pairs/host pool/staging")
    _err(call(staging=None), "NULL pairs/host pool/staging")
    _err(call(hk=FAKE + 4), "misaligned")
    _err(call(dev_pairs=FAKE + 4), "misaligned")
    assert call(nbytes=per_block - 1) == L.PA_ERR_WORKSPACE
    cache = L.KVCache(torch.zeros((4, 2, 16, 128), dtype=torch.float16),
                      torch.zeros((4, 2, 16, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="same shape"):
        L.pa_swap_blocks_dma(cache, torch.zeros((6, 2, 16, 128), dtype=torch.float16),
                             torch.zeros((3, 2, 16, 128), dtype=torch.float16), [[0, 0]], L.PA_SWAP_OUT,
                             torch.zeros(per_block, dtype=torch.uint8))

"""ctypes binding of libpagedattn (argument marshalling only).

Every computation happens in the HIP kernels behind the C-ABI declared in
``include/pagedattn.h``; this module only turns torch tensors into device
pointers and sizes, picks the stream, and turns a non-OK status into an
exception.  There is no fallback: if the shared library is missing the first
call raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_LAUNCH = range(5)
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_SWAP_OUT, PA_SWAP_IN = 0, 1
TORCH_TO_PA = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}

# every symbol include/pagedattn.h declares
EXPORTS = (
    "pa_reshape_and_cache", "pa_copy_blocks", "pa_swap_blocks", "pa_swap_blocks_dma", "pa_swap_staging_bytes",
    "pa_decode_workspace_bytes", "pa_paged_decode",
    "pa_paged_decode_noalloc", "pa_decode_grouped_workspace_bytes", "pa_paged_decode_grouped",
    "pa_paged_decode_append", "pa_paged_prefill", "pa_read_stream", "pa_read_tiles", "pa_check_copy_pairs",
    "pa_check_slot_mapping", "pa_check_block_tables", "pa_check_append_slots", "pa_check_prefill_rows", "pa_set_debug", "pa_get_debug", "pa_status_string", "pa_last_error", "pa_abi_version",
)


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class PaKVCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("dtype", ctypes.c_int),
    ]


_lib = None


def load_library(path: str) -> ctypes.CDLL:
    """Open a build of libpagedattn at ``path`` and declare its C signatures."""
    L = ctypes.CDLL(path)
    P, I32, I64P, I32P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    C = ctypes.POINTER(PaKVCache)
    L.pa_reshape_and_cache.argtypes = [C, P, P, I64P, I32, P]
    L.pa_copy_blocks.argtypes = [C, I64P, I32, P]
    L.pa_swap_blocks.argtypes = [C, P, P, I32, I64P, I32, ctypes.c_int, P]
    L.pa_swap_blocks_dma.argtypes = [C, P, P, I32, I64P, I64P, I32, ctypes.c_int, P, ctypes.c_size_t, P]
    L.pa_swap_staging_bytes.argtypes = [C, I32]
    L.pa_swap_staging_bytes.restype = ctypes.c_size_t
    L.pa_decode_workspace_bytes.argtypes = [C, I32, I32]
    L.pa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.pa_paged_decode.argtypes = [C, P, ctypes.c_int, P, I32P, I32, I32P, I32, I32, ctypes.c_float, P,
                                  ctypes.c_size_t, P]
    L.pa_paged_decode_noalloc.argtypes = [C, P, ctypes.c_int, P, I32P, I32, I32P, I32, I32, ctypes.c_float, P]
    L.pa_decode_grouped_workspace_bytes.argtypes = [C, I32, I32, I32]
    L.pa_decode_grouped_workspace_bytes.restype = ctypes.c_size_t
    L.pa_paged_decode_grouped.argtypes = [C, P, ctypes.c_int, P, I32P, I32, I32P, I32, I32, ctypes.c_float, I32,
                                          P, ctypes.c_size_t, P]
    L.pa_paged_decode_append.argtypes = [C, P, ctypes.c_int, P, P, P, P, I32P, I32, I32P, I32, I32,
                                         ctypes.c_float, I32, P, ctypes.c_size_t, P]
    L.pa_paged_prefill.argtypes = [C, P, ctypes.c_int, P, I32P, I32, I32P, I32P, I32, I32, I32,
                                   ctypes.c_float, P]
    L.pa_read_stream.argtypes = [P, ctypes.c_int64, P, P]
    L.pa_read_tiles.argtypes = [P, ctypes.c_int64, I32, I32P, I32, P, P]
    L.pa_check_copy_pairs.argtypes = [P, I32, I32, I32, I32]
    L.pa_check_slot_mapping.argtypes = [P, I32, ctypes.c_int64]
    L.pa_check_block_tables.argtypes = [P, I32, I32, P, I32, I32, I32]
    L.pa_check_append_slots.argtypes = [P, I32, I32, P, I32, P, I32]
    L.pa_check_prefill_rows.argtypes = [P, P, I32, I32]
    L.pa_set_debug.argtypes = [I32]
    L.pa_set_debug.restype = None
    L.pa_get_debug.argtypes = []
    L.pa_get_debug.restype = I32
    for fn in ("pa_reshape_and_cache", "pa_copy_blocks", "pa_swap_blocks", "pa_swap_blocks_dma", "pa_paged_decode",
               "pa_paged_decode_noalloc", "pa_paged_decode_grouped", "pa_paged_decode_append",
               "pa_paged_prefill", "pa_read_stream", "pa_read_tiles", "pa_check_copy_pairs", "pa_check_slot_mapping",
               "pa_check_block_tables", "pa_check_append_slots", "pa_check_prefill_rows"):
        getattr(L, fn).restype = ctypes.c_int
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_abi_version.argtypes = []
    L.pa_abi_version.restype = ctypes.c_int32
    return L


def lib() -> ctypes.CDLL:
    """Load the in-tree shared library (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_76_amd.build` "
            "(there is no non-HIP fallback)")
    _lib = load_library(LIB_PATH)
    return _lib


def _check(status: int) -> None:
    if status != PA_OK:
        L = lib()
        raise PagedAttnError(status, f"{L.pa_status_string(status).decode()}: {L.pa_last_error().decode()}")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _i32(**sizes) -> None:
    """Sizes the C-ABI takes as int32: refuse one that does not fit (ctypes
    would wrap it silently into another, smaller size, and the call would
    then cover only part of the caller's tensors)."""
    for name, v in sizes.items():
        if not -(1 << 31) <= int(v) < (1 << 31):
            raise ValueError(f"{name} = {int(v)} does not fit the C-ABI's int32")


@dataclass
class KVCache:
    """Caller-owned key/value pools ``[num_blocks][H][B][d]`` (torch tensors)."""

    k: torch.Tensor
    v: torch.Tensor

    @property
    def num_blocks(self) -> int:
        return self.k.shape[0]

    @property
    def num_heads(self) -> int:
        return self.k.shape[1]

    @property
    def block_size(self) -> int:
        return self.k.shape[2]

    @property
    def head_dim(self) -> int:
        return self.k.shape[3]

    @property
    def dtype(self) -> torch.dtype:
        return self.k.dtype

    def desc(self) -> PaKVCache:
        if self.k.shape != self.v.shape or self.k.dtype != self.v.dtype or self.k.dim() != 4:
            raise ValueError("k and v pools must both be [num_blocks][H][B][d] of one dtype")
        if not (self.k.is_contiguous() and self.v.is_contiguous()):
            raise ValueError("pools must be contiguous")
        _i32(num_blocks=self.num_blocks, num_heads=self.num_heads, head_dim=self.head_dim,
             block_size=self.block_size)
        return PaKVCache(self.k.data_ptr(), self.v.data_ptr(), self.num_blocks, self.num_heads,
                         self.head_dim, self.block_size, TORCH_TO_PA.get(self.dtype, -1))

    @staticmethod
    def empty(num_blocks: int, num_heads: int, block_size: int, head_dim: int,
              dtype: torch.dtype, device="cuda") -> "KVCache":
        shape = (num_blocks, num_heads, block_size, head_dim)
        return KVCache(torch.empty(shape, dtype=dtype, device=device),
                       torch.empty(shape, dtype=dtype, device=device))


def _device(cache: "KVCache", **tensors) -> None:
    """The pools are GPU tensors on the current device, and every device
    argument lives with them (a host or foreign pointer handed to a kernel
    would fault the GPU rather than raise)."""
    dev = cache.k.device
    if dev.type != "cuda" or cache.v.device != dev:
        raise ValueError(f"the k and v pools must be on one GPU, got {dev} and {cache.v.device}")
    if dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError(f"the pools are on {dev} but the current device is cuda:{torch.cuda.current_device()}")
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} must be on {dev}, got {t.device}")


def _contig(name: str, t: torch.Tensor, dtype=None) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def pa_reshape_and_cache(cache: KVCache, key: torch.Tensor, value: torch.Tensor,
                         slot_mapping: torch.Tensor, stream=None) -> None:
    """Write ``key, value [T][H][d]`` into the slots ``slot_mapping int64 [T]``."""
    _contig("key", key, cache.dtype)
    _contig("value", value, cache.dtype)
    _contig("slot_mapping", slot_mapping, torch.int64)
    T = slot_mapping.numel()
    if key.shape != (T, cache.num_heads, cache.head_dim) or value.shape != key.shape:
        raise ValueError(f"key/value must be [{T}][{cache.num_heads}][{cache.head_dim}]")
    _i32(T=T)
    _device(cache, key=key, value=value, slot_mapping=slot_mapping)
    d = cache.desc()
    _check(lib().pa_reshape_and_cache(ctypes.byref(d), _ptr(key), _ptr(value), _ptr(slot_mapping),
                                      T, _stream(stream)))


def pa_copy_blocks(cache: KVCache, pairs: torch.Tensor, stream=None) -> None:
    """Copy whole blocks ``dst <- src`` for each row of ``pairs int64 [n][2]``."""
    _contig("pairs", pairs, torch.int64)
    n = pairs.shape[0] if pairs.numel() else 0
    if pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2):
        raise ValueError("pairs must be [n][2]")
    _i32(pairs=n)
    _device(cache, pairs=pairs)
    d = cache.desc()
    _check(lib().pa_copy_blocks(ctypes.byref(d), _ptr(pairs) if n else None, n, _stream(stream)))


def pa_swap_blocks(cache: KVCache, host_k: torch.Tensor, host_v: torch.Tensor, pairs: torch.Tensor,
                   direction: int, stream=None) -> None:
    """Copy whole blocks between the device pools and pinned host pools
    ``[host_blocks][H][B][d]``; ``pairs int64 [n][2]`` on the device are
    (device, host) for PA_SWAP_OUT and (host, device) for PA_SWAP_IN."""
    _contig("pairs", pairs, torch.int64)
    for name, t in (("host_k", host_k), ("host_v", host_v)):
        _contig(name, t, cache.dtype)
        if t.dim() != 4 or t.shape[1:] != cache.k.shape[1:] or t.device.type != "cpu":
            raise ValueError(f"{name} must be a host tensor [blocks][H][B][d]")
    if host_v.shape != host_k.shape:
        # one block count bounds both host pools in the kernel
        raise ValueError(f"host_k {tuple(host_k.shape)} and host_v {tuple(host_v.shape)} must have the same shape")
    if pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2):
        raise ValueError("pairs must be [n][2]")
    n = pairs.shape[0] if pairs.numel() else 0
    _i32(pairs=n, host_blocks=host_k.shape[0])
    _device(cache, pairs=pairs)
    d = cache.desc()
    _check(lib().pa_swap_blocks(ctypes.byref(d), _ptr(host_k), _ptr(host_v), host_k.shape[0],
                                _ptr(pairs) if n else None, n, int(direction), _stream(stream)))


def swap_staging(cache: KVCache, blocks: int) -> torch.Tensor:
    """A device staging buffer for pa_swap_blocks_dma with room for
    ``blocks`` blocks of keys and values."""
    _i32(blocks=blocks)
    n = lib().pa_swap_staging_bytes(ctypes.byref(cache.desc()), blocks)
    if n == 0:
        raise ValueError(f"no staging size for {blocks} blocks")
    return torch.empty(n, dtype=torch.uint8, device=cache.k.device)


def pa_swap_blocks_dma(cache: KVCache, host_k: torch.Tensor, host_v: torch.Tensor, pairs, direction: int,
                       staging: torch.Tensor, stream=None, pairs_dev: torch.Tensor | None = None) -> None:
    """pa_swap_blocks with the host link driven by the copy engines:
    ``pairs int64 [n][2]`` in host memory (a numpy array or a CPU tensor),
    (device, host) for PA_SWAP_OUT and (host, device) for PA_SWAP_IN; their
    device copy ``pairs_dev`` is made here (synchronously) when not given.
    ``staging``: a device buffer from swap_staging()."""
    import numpy as np
    p = np.ascontiguousarray(pairs.numpy() if isinstance(pairs, torch.Tensor) else pairs, dtype=np.int64)
    if p.size and (p.ndim != 2 or p.shape[1] != 2):
        raise ValueError("pairs must be [n][2]")
    for name, t in (("host_k", host_k), ("host_v", host_v)):
        _contig(name, t, cache.dtype)
        if t.dim() != 4 or t.shape[1:] != cache.k.shape[1:] or t.device.type != "cpu":
            raise ValueError(f"{name} must be a host tensor [blocks][H][B][d]")
    if host_v.shape != host_k.shape:
        raise ValueError(f"host_k {tuple(host_k.shape)} and host_v {tuple(host_v.shape)} must have the same shape")
    _contig("staging", staging, torch.uint8)
    n = p.shape[0] if p.size else 0
    if pairs_dev is None:
        pairs_dev = torch.from_numpy(p.reshape(-1, 2)).to(cache.k.device)  # synchronous copy
        if stream is not None:
            pairs_dev.record_stream(stream)
    _i32(pairs=n, host_blocks=host_k.shape[0])
    _contig("pairs_dev", pairs_dev, torch.int64)
    if tuple(pairs_dev.shape) != (n, 2) and n:
        raise ValueError("pairs_dev must match pairs")
    _device(cache, pairs_dev=pairs_dev, staging=staging)
    d = cache.desc()
    _check(lib().pa_swap_blocks_dma(ctypes.byref(d), _ptr(host_k), _ptr(host_v), host_k.shape[0],
                                    _ptr(pairs_dev) if n else None,
                                    p.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)) if n else None, n,
                                    int(direction), _ptr(staging), staging.numel(), _stream(stream)))


def pa_decode_workspace_bytes(cache: KVCache, S: int, max_context_len: int) -> int:
    _i32(S=S, max_context_len=max_context_len)
    d = cache.desc()
    n = lib().pa_decode_workspace_bytes(ctypes.byref(d), S, max_context_len)
    if n == ctypes.c_size_t(-1).value:
        raise PagedAttnError(PA_ERR_UNSUPPORTED, lib().pa_last_error().decode())
    return n


def decode_workspace(cache: KVCache, S: int, max_context_len: int) -> torch.Tensor | None:
    """Allocate (with torch) the scratch that :func:`pa_paged_decode` needs."""
    n = pa_decode_workspace_bytes(cache, S, max_context_len)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=cache.k.device)


def pa_paged_decode(cache: KVCache, out: torch.Tensor, query: torch.Tensor,
                    block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                    scale: float, workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step: ``out [S][H][d]`` (cache dtype or float32)."""
    _contig("query", query, cache.dtype)
    _contig("out", out)
    _contig("block_tables", block_tables, torch.int32)
    _contig("context_lens", context_lens, torch.int32)
    S = query.shape[0]
    if query.shape != (S, cache.num_heads, cache.head_dim) or out.shape != query.shape:
        raise ValueError("query/out must be [S][H][d]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S][max_blocks], context_lens [S]")
    _i32(S=S, max_blocks_per_seq=block_tables.shape[1], max_context_len=max_context_len)
    _device(cache, out=out, query=query, block_tables=block_tables, context_lens=context_lens, workspace=workspace)
    d = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_paged_decode(ctypes.byref(d), _ptr(out), TORCH_TO_PA.get(out.dtype, -1), _ptr(query),
                                 _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S,
                                 int(max_context_len), float(scale), _ptr(workspace), ws_bytes,
                                 _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20  # PA_NOALLOC_SCRATCH_BYTES of include/pagedattn.h


def pa_paged_decode_noalloc(cache: KVCache, out: torch.Tensor, query: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                            scale: float, stream=None) -> torch.Tensor:
    """:func:`pa_paged_decode` with the library's own scratch array instead
    of a workspace (nothing is allocated; calls overlapping on one GPU race)."""
    _contig("query", query, cache.dtype)
    _contig("out", out)
    _contig("block_tables", block_tables, torch.int32)
    _contig("context_lens", context_lens, torch.int32)
    S = query.shape[0]
    if query.shape != (S, cache.num_heads, cache.head_dim) or out.shape != query.shape:
        raise ValueError("query/out must be [S][H][d]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S][max_blocks], context_lens [S]")
    _i32(S=S, max_blocks_per_seq=block_tables.shape[1], max_context_len=max_context_len)
    _device(cache, out=out, query=query, block_tables=block_tables, context_lens=context_lens)
    d = cache.desc()
    _check(lib().pa_paged_decode_noalloc(ctypes.byref(d), _ptr(out), TORCH_TO_PA.get(out.dtype, -1), _ptr(query),
                                         _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S,
                                         int(max_context_len), float(scale), _stream(stream)))
    return out


def pa_decode_grouped_workspace_bytes(cache: KVCache, S: int, max_context_len: int, group_size: int) -> int:
    _i32(S=S, max_context_len=max_context_len, group_size=group_size)
    d = cache.desc()
    n = lib().pa_decode_grouped_workspace_bytes(ctypes.byref(d), S, max_context_len, group_size)
    if n == ctypes.c_size_t(-1).value:
        raise PagedAttnError(PA_ERR_INVALID_ARG, lib().pa_last_error().decode())
    return n


def decode_grouped_workspace(cache: KVCache, S: int, max_context_len: int, group_size: int) -> torch.Tensor | None:
    """Allocate (with torch) the scratch that :func:`pa_paged_decode_grouped` needs."""
    n = pa_decode_grouped_workspace_bytes(cache, S, max_context_len, group_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=cache.k.device)


def pa_paged_decode_grouped(cache: KVCache, out: torch.Tensor, query: torch.Tensor,
                            block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                            scale: float, group_size: int, workspace: torch.Tensor | None = None,
                            stream=None) -> torch.Tensor:
    """Decode with rows taken ``group_size`` at a time; blocks shared by a
    whole group are read once.  Same result as :func:`pa_paged_decode`."""
    _contig("query", query, cache.dtype)
    _contig("out", out)
    _contig("block_tables", block_tables, torch.int32)
    _contig("context_lens", context_lens, torch.int32)
    S = query.shape[0]
    if query.shape != (S, cache.num_heads, cache.head_dim) or out.shape != query.shape:
        raise ValueError("query/out must be [S][H][d]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S][max_blocks], context_lens [S]")
    _i32(S=S, max_blocks_per_seq=block_tables.shape[1], max_context_len=max_context_len)
    _device(cache, out=out, query=query, block_tables=block_tables, context_lens=context_lens, workspace=workspace)
    d = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_paged_decode_grouped(ctypes.byref(d), _ptr(out), TORCH_TO_PA.get(out.dtype, -1), _ptr(query),
                                         _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S,
                                         int(max_context_len), float(scale), int(group_size), _ptr(workspace),
                                         ws_bytes, _stream(stream)))
    return out


def pa_paged_decode_append(cache: KVCache, out: torch.Tensor, query: torch.Tensor, key: torch.Tensor,
                           value: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, scale: float, group_size: int = 1,
                           workspace: torch.Tensor | None = None, stream=None,
                           cow_src: torch.Tensor | None = None) -> torch.Tensor:
    """Store each row's newest token (``key``/``value`` [S][H][d], position
    ``context_lens[s] - 1``) in the cache and decode, in one launch.  With
    ``cow_src`` (int32 [S], -1 = none) the row's newest-token block first
    receives a copy of block ``cow_src[s]`` in the same launch.  Same cache as
    :func:`pa_copy_blocks` (those pairs), :func:`pa_reshape_and_cache`, and the
    output of :func:`pa_paged_decode` (``group_size`` 1) or
    :func:`pa_paged_decode_grouped` after them.  ``workspace``: see
    :func:`decode_grouped_workspace` with the same ``group_size``."""
    _contig("query", query, cache.dtype)
    _contig("key", key, cache.dtype)
    _contig("value", value, cache.dtype)
    _contig("out", out)
    _contig("block_tables", block_tables, torch.int32)
    _contig("context_lens", context_lens, torch.int32)
    S = query.shape[0]
    if query.shape != (S, cache.num_heads, cache.head_dim) or out.shape != query.shape:
        raise ValueError("query/out must be [S][H][d]")
    if key.shape != query.shape or value.shape != query.shape:
        raise ValueError("key/value must be [S][H][d], one new token per row")
    if cow_src is not None:
        _contig("cow_src", cow_src, torch.int32)
        if cow_src.shape != (query.shape[0],):
            raise ValueError("cow_src must be [S]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S][max_blocks], context_lens [S]")
    _i32(S=S, max_blocks_per_seq=block_tables.shape[1], max_context_len=max_context_len)
    _device(cache, out=out, query=query, key=key, value=value, block_tables=block_tables,
            context_lens=context_lens, workspace=workspace, cow_src=cow_src)
    d = cache.desc()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pa_paged_decode_append(ctypes.byref(d), _ptr(out), TORCH_TO_PA.get(out.dtype, -1), _ptr(query),
                                        _ptr(key), _ptr(value), _ptr(cow_src), _ptr(block_tables),
                                        block_tables.shape[1],
                                        _ptr(context_lens), S, int(max_context_len), float(scale), int(group_size),
                                        _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def pa_paged_prefill(cache: KVCache, out: torch.Tensor, query: torch.Tensor,
                     block_tables: torch.Tensor, cu_q_lens: torch.Tensor, context_lens: torch.Tensor,
                     max_q_len: int, max_context_len: int, scale: float, stream=None) -> torch.Tensor:
    """Causal prefill: ``out [sum q][H][d]`` (cache dtype or float32)."""
    _contig("query", query, cache.dtype)
    _contig("out", out)
    _contig("block_tables", block_tables, torch.int32)
    _contig("cu_q_lens", cu_q_lens, torch.int32)
    _contig("context_lens", context_lens, torch.int32)
    S = context_lens.shape[0]
    if query.dim() != 3 or query.shape[1:] != (cache.num_heads, cache.head_dim):
        raise ValueError(f"query must be [rows][{cache.num_heads}][{cache.head_dim}]")
    if (cu_q_lens.shape != (S + 1,) or out.shape != query.shape or block_tables.dim() != 2
            or block_tables.shape[0] != S):
        raise ValueError("cu_q_lens must be [S+1], block_tables [S][max_blocks], out like query")
    _i32(S=S, max_blocks_per_seq=block_tables.shape[1], max_q_len=max_q_len,
         max_context_len=max_context_len, rows=query.shape[0])
    _device(cache, out=out, query=query, block_tables=block_tables, cu_q_lens=cu_q_lens, context_lens=context_lens)
    if S and get_debug():
        # the rows of sequence s are cu_q_lens[s] .. cu_q_lens[s+1]-1 of query
        # and out; the C-ABI is not given their count, so it is checked here
        # (a device read, like the library's own debug-mode index checks)
        total = int(cu_q_lens[S].item())
        if total > query.shape[0]:
            raise PagedAttnError(PA_ERR_INVALID_ARG, f"cu_q_lens[S] = {total} exceeds the {query.shape[0]} "
                                 "rows of query and out")
    d = cache.desc()
    _check(lib().pa_paged_prefill(ctypes.byref(d), _ptr(out), TORCH_TO_PA.get(out.dtype, -1), _ptr(query),
                                  _ptr(block_tables), block_tables.shape[1], _ptr(cu_q_lens),
                                  _ptr(context_lens), S, int(max_q_len), int(max_context_len),
                                  float(scale), _stream(stream)))
    return out


# ---- measurement reads (not part of the method) ----------------------------------

def _on_gpu(**tensors) -> None:
    for name, t in tensors.items():
        if t.device.type != "cuda" or (t.device.index is not None and t.device.index != torch.cuda.current_device()):
            raise ValueError(f"{name} must be on the current GPU, got {t.device}")


def pa_read_stream(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read all of ``buf`` once (the achievable streaming-read rate)."""
    _on_gpu(buf=buf, sink=sink)
    _contig("buf", buf)
    _check(lib().pa_read_stream(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def pa_read_tiles(buf: torch.Tensor, tile_bytes: int, tiles: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Read the tiles ``buf`` + ``tiles[i]`` * ``tile_bytes`` (the block-table access pattern, no arithmetic)."""
    _on_gpu(buf=buf, tiles=tiles, sink=sink)
    _contig("buf", buf)
    tiles = _contig("tiles", tiles, torch.int32)
    nbytes = buf.numel() * buf.element_size()
    _i32(tiles=tiles.numel())
    num_tiles = min(nbytes // int(tile_bytes), (1 << 31) - 1)  # a bound on the (int32) tile ids
    _check(lib().pa_read_tiles(_ptr(buf), int(tile_bytes), num_tiles, _ptr(tiles), tiles.numel(),
                               _ptr(sink), _stream(stream)))


# ---- index-precondition checks (host arrays; no device is touched) ---------------

def _host_array(a, dtype):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def check_copy_pairs(pairs, src_blocks: int, dst_blocks: int, same_pool: bool = True) -> None:
    """Raise if the (src, dst) pairs break pa_copy_blocks' / pa_swap_blocks'
    preconditions (ids in range, distinct destinations, no destination that
    is also a source when both sides are one pool)."""
    import numpy as np
    a, p = _host_array(np.asarray(pairs).reshape(-1, 2), np.int64)
    _check(lib().pa_check_copy_pairs(p, a.shape[0], int(src_blocks), int(dst_blocks), int(bool(same_pool))))


def check_slot_mapping(slots, num_slots: int) -> None:
    """Raise if two tokens share a slot or a slot lies outside the pool."""
    import numpy as np
    a, p = _host_array(slots, np.int64)
    _check(lib().pa_check_slot_mapping(p, a.size, int(num_slots)))


def check_block_tables(tables, context_lens, max_context_len: int, block_size: int, num_blocks: int) -> None:
    """Raise if a context length or a table entry it uses is out of range."""
    import numpy as np
    t, pt = _host_array(tables, np.int32)
    lens, pl = _host_array(context_lens, np.int32)
    if t.ndim != 2 or t.shape[0] != lens.size:
        raise ValueError("tables must be [S][max_blocks] and context_lens [S]")
    _check(lib().pa_check_block_tables(pt, lens.size, t.shape[1], pl, int(max_context_len), int(block_size),
                                       int(num_blocks)))


def check_append_slots(tables, context_lens, block_size: int, cow_src=None, num_blocks: int | None = None) -> None:
    """Raise if two rows' newest tokens share a slot or another row reads one,
    or (with ``cow_src``, which needs ``num_blocks``) a folded-in copy breaks
    its preconditions."""
    import numpy as np
    t, pt = _host_array(tables, np.int32)
    lens, pl = _host_array(context_lens, np.int32)
    if t.ndim != 2 or t.shape[0] != lens.size:
        raise ValueError("tables must be [S][max_blocks] and context_lens [S]")
    pc, nb = None, 0
    if cow_src is not None:
        if num_blocks is None:
            raise ValueError("num_blocks is needed with cow_src")
        cw, pc = _host_array(cow_src, np.int32)
        if cw.shape != (lens.size,):
            raise ValueError("cow_src must be [S]")
        nb = int(num_blocks)
    _check(lib().pa_check_append_slots(pt, lens.size, t.shape[1], pl, int(block_size), pc, nb))


def check_prefill_rows(cu_q_lens, context_lens, max_q_len: int) -> None:
    """Raise if the query ranges of a prefill call are malformed."""
    import numpy as np
    cu, pc = _host_array(cu_q_lens, np.int32)
    lens, pl = _host_array(context_lens, np.int32)
    if cu.size != lens.size + 1:
        raise ValueError("cu_q_lens must be [S+1]")
    _check(lib().pa_check_prefill_rows(pc, pl, lens.size, int(max_q_len)))


def set_debug(on: bool) -> None:
    """Check index preconditions (host copies of the index arrays) before every launch."""
    lib().pa_set_debug(1 if on else 0)


def get_debug() -> bool:
    return bool(lib().pa_get_debug())

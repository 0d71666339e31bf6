"""CPU oracle for paged KV-cache attention — TEST INFRASTRUCTURE ONLY.

This package is the independent reference the HIP path in
``paged_kv_cache_76_amd`` is checked against.  It is plain, slow, obviously-correct NumPy in
float64 and shares no code with the GPU library: it never sees a kernel, a
header, a helper or a constant generator of the product, and the product never
imports it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.

Sources (the three web pages on vLLM / PagedAttention):

* "vLLM / PagedAttention — 把 LLM 服务的瓶颈从显存碎片里救出来"
  (awesome.papernotes.org), "方法详解": key design 1 (exact attention, eq. 1,
  and its block-wise form, eq. 2), key design 2 (block table, on-demand
  allocation, tail-waste bound eq. 3), key design 3 (sharing, reference
  counts, copy-on-write, the physical-block count eq. 4 and the
  ``append_token`` pseudocode), key design 5 (fused reshape/write, block-read
  attention, batched block copy).
* "vLLM" notes (formulaic.cloudchewie.com), "PagedAttention 原理" (the
  7-token, B=4 worked example) and "在不同解码策略下的效果" (parallel-sampling
  copy-on-write, beam search).
* "vLLM / PagedAttention (SOSP 2023)" system-design guide (upskillscore),
  sections 03 and 04.

Modules:

* :mod:`oracle.attention` — decode and causal prefill attention over the
  logically contiguous history (pinned: closed forms, a library SDPA in
  float64, the block-wise eq. 2, brute force on tiny inputs).
* :mod:`oracle.cache` — what a slot-mapped cache write and a batched block
  copy must leave in the pools (pinned: read-back through block tables,
  untouched-bytes invariants).
* :mod:`oracle.block_model` — a dictionary model of the block manager
  (pinned: both worked examples of the pages, eq. 3 and eq. 4 identities,
  brute-force enumeration of short operation sequences).

Every function in this package has at least one pin in ``tests/``; none is
"parity unpinned".
"""

from . import attention, block_model, cache  # noqa: F401

"""CPU oracle for the paged-KV-cache hot path: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The library under
``paged_kv_cache_130_amd`` never imports it. The two share no code; only the
seeded generators in ``workloads`` feed both.

This is a plain, slow, obviously correct NumPy implementation in float64. It
reads the stored bits of every input (fp16, bf16, e4m3, float32 scales) and
decodes them exactly, so that rounding of the inputs is never counted as
kernel error. It computes:

* ``numerics``: exact decoding of fp16, bf16 and OCP e4m3 bytes.
* ``paging``: blocks per sequence, slot integers, the cache-view byte
  address, and the stride rules of the layer-outer and block-outer layouts.
* ``cache_write``: the ``reshape_and_cache`` scatter, as bytes.
* ``quant``: quantize-on-write of the DSA dual cache rows (bf16 in, packed
  fp8 rows with float32 group scales out), then the same scatter.
* ``attention``: paged decode (dense and grouped heads), causal chunks over
  paged context, MLA latent decode, and the log-sum-exp merge of
  split-context partials.
* ``dsa``: the sparse path over the DSA dual cache: lightning-indexer scores
  from the indexer rows, the top-k selection, and MLA decode over the
  selected slots.

Sources. These are the four pages on vLLM's KV cache, cited by title:

* "deep dive into vLLM 05: KV cache memory core" (arganzheng.life)
* "vLLM KV Cache Layout 可视化" (riverclouds.net)
* "KV Cache 与推理服务内存管理" (pinghaoyang.com.cn)
* "vLLM 技术内幕——像操作系统管理内存一样管理 KV 缓存" (openeuler.csdn.net)

Every function is pinned by a CPU test against something other than itself:
the pages' worked numbers, closed forms, torch library routines, or brute
force. No function is parity-unpinned.
"""

from . import numerics, paging, cache_write, attention, quant, dsa  # noqa: F401

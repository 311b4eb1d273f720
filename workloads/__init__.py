"""Seeded synthetic inputs for the paged-KV-cache hot path.

This module is shared by the tests, the oracle checks and the bench. It holds
no arithmetic of the attention or of the cache write: it draws values, picks
physical blocks and lays out what an out-of-scope scheduler would hand to the
kernels. That means context lengths, block tables and the ``slot_mapping``
integers. The kernels split those integers back into block and position and
apply the cache views. The oracle does the same independently.

Workload recipes. Each one stands in for a workload the pages describe:

* ``tiny``: 4 sequences with contexts {1, 17, 130, 300}, 8 heads of 128, fp16,
  block size 16, a pool of 64 blocks.
* ``mha13b``: a 13B-shaped MHA decode layer. Batch 64, contexts uniform in
  [128, 2048], 40 heads of 128, fp16, block size 16, a pool of 12288 blocks.
  The 13B model's ~800 KB of KV per token is on the "vLLM 技术内幕" page, §1.
* ``gqa_prefix``: GQA decode with a shared 2000-token (125-block) system
  prompt. Batch 256, 32 query / 8 KV heads, bf16. Each private suffix is
  lognormal with median 300 and sigma 1.0, rounded, clipped to [1, 6000].
  The 125-block prompt is on the "deep dive into vLLM 05" page, §3.1.
* ``long_mixed``: 8 decodes at 32768 tokens (split-context partitions of
  512), plus a 3000-token prompt cut into 2048 + 952 causal chunks beside two
  decodes A and B. 32/8 heads, bf16. The chunking example is on the
  "vLLM 技术内幕" page, §3.2.
* ``dsa_mla``: the DSA dual cache in block-outer BLHNC layout. 2 layers,
  block size 64, 656-byte MLA rows and 132-byte indexer rows, then MLA decode
  with 128 heads on one latent head. The layout is the worked example of the
  "vLLM KV Cache Layout 可视化" page. The sparse path adds, per decode token, 64
  lightning-indexer queries of 128 bf16 values with float32 head weights
  N(0, 1/64), and selects the top 2048 tokens (the page gives neither the head
  count nor k; these are DeepSeek's published indexer settings).

Every draw uses NumPy's PCG64 with a fixed seed per workload. Values are
N(0, 1) float32, rounded to the storage type with round-to-nearest-even by
NumPy (fp16) or torch (bf16, float8_e4m3fn) library casts.
"""

from .gen import (  # noqa: F401
    INT32_PAD,
    SEEDS,
    WORKLOADS,
    DenseCase,
    MlaCase,
    ChunkCase,
    allocate_block_tables,
    draw_bits,
    draw_context_lens,
    draw_mla_rows,
    draw_indexer_rows,
    draw_index_queries,
    f16_nan_bits,
    bf16_nan_bits,
    make_dense_case,
    make_mla_case,
    make_chunk_case,
    slots_for_positions,
    workload,
)

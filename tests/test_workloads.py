"""Sanity of the seeded generators (shapes, recipe statistics, determinism)."""

import numpy as np
import torch

import workloads
from oracle import paging as P


def test_tiny_case_shapes_and_poisoned_unused_blocks():
    c = workloads.make_dense_case("tiny")
    assert c.k_pool.shape == (64, 16, 8, 128) and c.q.shape == (4, 8, 128)
    assert c.context_lens.tolist() == [1, 17, 130, 300]
    need = sum(P.blocks_needed(n, 16) for n in c.context_lens)
    assert need == 31
    used = set(c.block_tables[c.block_tables != workloads.INT32_PAD].tolist())
    assert len(used) == 31
    kp = c.k_pool.view(torch.float16)
    for b in range(64):
        assert bool(torch.isnan(kp[b]).all()) == (b not in used)
    again = workloads.make_dense_case("tiny")
    assert torch.equal(again.k_pool, c.k_pool) and np.array_equal(again.block_tables, c.block_tables)


def test_mha13b_recipe_without_pools():
    c = workloads.make_dense_case("mha13b", with_pools=False)
    ctx = c.context_lens
    assert len(ctx) == 64 and ctx.min() >= 128 and ctx.max() <= 2048
    assert (ctx % 16 != 0).any()                       # some last blocks are partial
    assert c.num_blocks == 12288 and c.row_bytes == 10240


def test_gqa_prefix_recipe_shares_125_blocks():
    c = workloads.make_dense_case("gqa_prefix", with_pools=False)
    assert len(c.context_lens) == 256 and (c.context_lens >= 2001).all() and (c.context_lens <= 8000).all()
    first = c.block_tables[:, :125]
    assert (first == first[0]).all()
    med = np.median(c.context_lens - 2000)
    assert 200 < med < 450
    cp = workloads.make_dense_case("gqa_prefix", with_pools=False, copied_prefix=True)
    assert len(np.unique(cp.block_tables[:, :125])) == 256 * 125


def test_long_mixed_steps():
    s1 = workloads.make_chunk_case(step=1, with_pools=False)
    s2 = workloads.make_chunk_case(step=2, with_pools=False)
    assert s1.total_q == 8 + 2 + 2048 and s2.total_q == 8 + 2 + 952
    assert s1.seq_lens.tolist()[-1] == 2048 and s2.seq_lens.tolist()[-1] == 3000
    assert np.array_equal(s1.block_tables, s2.block_tables)


def test_mla_rows_layout():
    r = workloads.draw_mla_rows(1, 5)
    assert r.shape == (5, 656) and r.dtype == torch.uint8
    lat = r[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float32).reshape(5, 4, 128)
    assert (lat.abs().amax(dim=2) == 448).all()        # each 128-group reaches the e4m3 maximum
    x = workloads.draw_indexer_rows(2, 3)
    assert x.shape == (3, 132)

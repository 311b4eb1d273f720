"""Pins for oracle.paging against the pages' worked numbers (tests/golden/*.json)."""

import json
import os

import numpy as np
import pytest

from oracle import paging as P
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_block_counts_from_page():
    g = load("block_counts.json")
    bs = g["block_size"]
    for c in g["cases"]:
        assert P.blocks_needed(c["tokens"], bs) == c["blocks"]
        if "full_blocks" in c:
            assert P.full_blocks(c["tokens"], bs) == c["full_blocks"]
        if "tokens_in_last_block" in c:
            last = c["tokens"] - (P.blocks_needed(c["tokens"], bs) - 1) * bs
            assert last == c["tokens_in_last_block"]


def test_slot_322_from_page():
    g = load("layout_worked_example.json")
    bs = g["block_size"]
    table = [11, 7, g["block_table_entry"], 3]          # only entry 2 is given by the page
    lb, off = P.logical_block_and_offset(g["token_position"], bs)
    assert (lb, off) == (g["logical_block"], g["in_block_position"])
    slot = P.slot_of(table, g["token_position"], bs)
    assert slot == g["slot"]
    assert P.split_slot(slot, bs) == (g["block_table_entry"], g["in_block_position"])


def test_blhnc_pages_views_and_addresses_from_page():
    g = load("layout_worked_example.json")
    bs, nl = g["block_size"], g["num_layers"]
    assert sum(g["mla_row_bytes_parts"].values()) == g["mla_row_bytes"]
    assert sum(g["indexer_row_bytes_parts"].values()) == g["indexer_row_bytes"]
    assert P.page_bytes(bs, g["mla_row_bytes"]) == g["mla_page_bytes"]
    assert P.page_bytes(bs, g["indexer_row_bytes"]) == g["indexer_page_bytes"]
    views, total = P.block_outer_views([("mla", g["mla_row_bytes"], nl), ("indexer", g["indexer_row_bytes"], nl)], bs)
    assert total == g["block_bytes"]
    for name in ("mla", "indexer"):
        v = views[name]
        want = g["views"][name]
        assert (v.offset, v.layer_stride, v.block_stride, v.row_bytes) == (
            want["offset"], want["layer_stride"], want["block_stride"], want["row_bytes"])
    # in-block boundaries: MLA L0 | MLA L1 | IDX L0 | IDX L1 | end
    bounds = [P.address(views["mla"], 0, 0, 0), P.address(views["mla"], 1, 0, 0),
              P.address(views["indexer"], 0, 0, 0), P.address(views["indexer"], 1, 0, 0),
              P.address(views["mla"], 0, 1, 0)]
    assert bounds == g["in_block_boundaries"]
    b, pos = P.split_slot(g["slot"], bs)
    for name in ("mla", "indexer"):
        assert P.address(views[name], g["layer"], b, pos) == sum(g["layer1_address_terms"][name])
    assert P.address(views["mla"], 1, b, pos) == 547616
    assert P.address(views["indexer"], 1, b, pos) == 597000


def test_layer_outer_stride_rule_and_single_block_invariant():
    caches = [("mla", 656, 2), ("indexer", 132, 2)]
    lo = P.layer_outer_views(caches, 64, num_blocks=9216)
    assert lo["mla"].block_stride == 41984 and lo["mla"].layer_stride == 41984 * 9216
    assert lo["indexer"].block_stride == 8448 and lo["indexer"].layer_stride == 8448 * 9216
    assert lo["indexer"].offset == 2 * 41984 * 9216
    # With one block, layer-outer and block-outer place every row at the same byte.
    lo1 = P.layer_outer_views(caches, 64, num_blocks=1)
    bo1, _ = P.block_outer_views(caches, 64)
    for name in ("mla", "indexer"):
        for layer in range(2):
            for pos in (0, 17, 63):
                assert P.address(lo1[name], layer, 0, pos) == P.address(bo1[name], layer, 0, pos)


def test_views_tile_the_allocation_without_overlap():
    # Every (cache, layer, block, position) row occupies distinct bytes, and the rows cover the block exactly.
    caches = [("mla", 656, 2), ("indexer", 132, 2)]
    bo, total = P.block_outer_views(caches, 4)
    nb = 3
    cover = np.zeros(total * nb, dtype=np.int32)
    for name, row, nl in caches:
        for layer in range(nl):
            for b in range(nb):
                for pos in range(4):
                    a = P.address(bo[name], layer, b, pos)
                    cover[a:a + row] += 1
    assert (cover == 1).all()


def test_footprints_from_pages():
    g = load("footprints.json")
    m = g["mha13b"]
    per_token = m["num_layers"] * 2 * P.dense_row_bytes(m["num_kv_heads"], m["head_dim"], m["elem_bytes"])
    assert per_token == m["kib_per_token"] * 1024
    assert abs(per_token * m["tokens"] / 1e9 - m["gb_per_sequence_approx"]) < 0.1
    q = g["gqa8"]
    assert 2 * P.dense_row_bytes(q["num_kv_heads"], q["head_dim"], q["elem_bytes"]) == q["kib_per_token_per_layer"] * 1024


def test_generator_slots_agree_with_oracle_slot_of():
    # The generator composes slots as the out-of-scope scheduler would; check it against the oracle.
    rng = np.random.Generator(np.random.PCG64(5))
    ctx = [1, 17, 130, 300]
    tables, _ = workloads.allocate_block_tables(rng, ctx, 16, 64)
    for b, n in enumerate(ctx):
        pos = np.arange(n)
        s = workloads.slots_for_positions(tables[b], pos, 16)
        assert [P.slot_of(tables[b], p, 16) for p in pos] == s.tolist()
        assert len(set(s.tolist())) == n
    used = tables[tables != workloads.INT32_PAD]
    assert len(np.unique(used)) == len(used) == sum(P.blocks_needed(n, 16) for n in ctx)


@pytest.mark.parametrize("bs", [16, 64])
def test_slot_split_round_trip(bs):
    rng = np.random.default_rng(bs)
    for _ in range(200):
        table = rng.permutation(1000)[:50]
        pos = int(rng.integers(0, 50 * bs))
        b, off = P.split_slot(P.slot_of(table, pos, bs), bs)
        assert b == table[pos // bs] and off == pos % bs

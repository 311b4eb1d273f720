"""Pins for oracle.cache_write: exact by construction, checked by round trip and sentinels."""

import numpy as np

from oracle import attention as A
from oracle import cache_write as W
from oracle import paging as P
import workloads

SENTINEL = 0xA5


def test_round_trip_and_untouched_bytes():
    rng = np.random.Generator(np.random.PCG64(11))
    bs, nb, row = 16, 40, 96
    view = P.CacheView(offset=0, layer_stride=0, block_stride=bs * row, row_bytes=row)
    image = np.full(nb * bs * row, SENTINEL, dtype=np.uint8)
    ctx = [5, 16, 33]
    tables, _ = workloads.allocate_block_tables(rng, ctx, bs, nb)
    written = np.zeros_like(image, dtype=bool)
    for b, n in enumerate(ctx):
        rows = rng.integers(0, 256, size=(n, row), dtype=np.uint8)
        rows[rows == SENTINEL] = 0
        slots = workloads.slots_for_positions(tables[b], np.arange(n), bs)
        image = W.reshape_and_cache(image, rows, slots, view, 0, bs)
        back = A.gather_rows(image, view, 0, tables[b], n, bs)
        assert np.array_equal(back, rows)
        for s in slots:
            a = P.address(view, 0, *P.split_slot(s, bs))
            written[a:a + row] = True
    assert (image[~written] == SENTINEL).all()
    assert (image[written] != SENTINEL).all()


def test_negative_slots_are_padding():
    view = P.CacheView(offset=8, layer_stride=0, block_stride=64, row_bytes=16)
    image = np.zeros(8 + 64 * 2, dtype=np.uint8)
    rows = np.arange(32, dtype=np.uint8).reshape(2, 16) + 1
    out = W.reshape_and_cache(image, rows, [-1, 5], view, 0, 4)
    assert out[8 + 64 * 1 + 16 * 1: 8 + 64 + 32].tolist() == rows[1].tolist()
    assert out.sum() == rows[1].astype(int).sum()


def test_dual_view_write_lands_at_page_addresses():
    # One slot_mapping, two views (MLA 656 B rows, indexer 132 B rows), layer 1 of the BLHNC example.
    bs = 64
    views, block = P.block_outer_views([("mla", 656, 2), ("indexer", 132, 2)], bs)
    nb = 8
    image = np.full(nb * block, SENTINEL, dtype=np.uint8)
    mla = np.full((1, 656), 0x11, dtype=np.uint8)
    idx = np.full((1, 132), 0x22, dtype=np.uint8)
    image = W.reshape_and_cache(image, mla, [322], views["mla"], 1, bs)
    image = W.reshape_and_cache(image, idx, [322], views["indexer"], 1, bs)
    assert (image[547616:547616 + 656] == 0x11).all()
    assert (image[597000:597000 + 132] == 0x22).all()
    assert (image == 0x11).sum() == 656 and (image == 0x22).sum() == 132


def test_copy_blocks_is_copy_on_write_for_a_shared_prefix():
    # "vLLM 技术内幕" §2.2: sequences share a prefix's physical blocks (ref_cnt > 1); copy-on-write gives
    # a sequence its own copy. After copying the shared blocks to fresh ones and pointing the
    # sequence's table at them, every row read through the new table equals the row read through the
    # old one, decode is unchanged, and no byte outside the destination pages moved.
    rng = np.random.Generator(np.random.PCG64(5))
    bs, nb, hkv, d = 16, 48, 2, 8
    row = hkv * d * 2
    for layout in ("layer", "block"):
        L = 3
        if layout == "layer":
            view = P.CacheView(0, nb * bs * row, bs * row, row)
            size = L * nb * bs * row
        else:
            view = P.CacheView(0, bs * row, L * bs * row, row)
            size = nb * L * bs * row
        # finite fp16 bit patterns in [0, 1), so decode outputs compare exactly
        image = rng.integers(0, 0x3C00, size=size // 2, dtype=np.uint16).view(np.uint8)
        shared = [3, 17, 8]                 # a 3-block prefix shared by two sequences
        fresh = [40, 41, 42]
        table_a = np.array(shared + [20], dtype=np.int64)
        out = W.copy_blocks(image, view, list(zip(shared, fresh)), L, bs)
        table_b = np.array(fresh + [20], dtype=np.int64)
        for layer in range(L):
            assert np.array_equal(A.gather_rows(out, view, layer, table_b, 60, bs),
                                  A.gather_rows(image, view, layer, table_a, 60, bs))
        moved = np.zeros(size, dtype=bool)
        for blk in fresh:
            for layer in range(L):
                a = P.address(view, layer, blk, 0)
                moved[a:a + bs * row] = True
        assert np.array_equal(out[~moved], image[~moved])
    # decode through either table is the same (K = V = the same rows here)
    q = rng.integers(0, 0x3C00, size=(1, 2, d)).astype(np.uint16)
    for tab in (table_a, table_b):
        assert tab.shape == (4,)
    ka = A.paged_decode(q, "f16", image, view, image, view, 1, table_a[None], [60], bs, hkv, d, 0.3)
    kb = A.paged_decode(q, "f16", out, view, out, view, 1, table_b[None], [60], bs, hkv, d, 0.3)
    assert np.array_equal(ka, kb)

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

"""The ``reshape_and_cache`` scatter, as bytes.

Sources:
* "vLLM KV Cache Layout 可视化", kernel section: the write kernel splits the
  slot into block = slot / block_size and position = slot % block_size. It
  then writes at cache + block*block_stride + position*row width, where the
  view's start already includes offset + layer*layer_stride.
* "vLLM 技术内幕", §2.1: write_to_paged_cache hands new K/V to the fused
  reshape_and_cache operator.
* "KV Cache 与推理服务内存管理", decode pseudocode: the new token's K/V go to
  (physical block, offset in block).

Readings where the pages are silent: a negative slot marks a padding token
and is skipped. Two tokens with the same slot in one call are a caller error
(asserted here).
"""

from __future__ import annotations

import numpy as np

from .paging import CacheView, address, split_slot


def reshape_and_cache(image: np.ndarray, rows: np.ndarray, slot_mapping, view: CacheView, layer: int,
                      block_size: int) -> np.ndarray:
    """Return a copy of ``image`` (uint8) with row t of ``rows`` written at slot_mapping[t]'s address."""
    out = np.array(image, dtype=np.uint8, copy=True)
    rows = np.asarray(rows, dtype=np.uint8)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    assert rows.ndim == 2 and rows.shape[1] == view.row_bytes and rows.shape[0] == slots.shape[0]
    valid = slots[slots >= 0]
    assert len(np.unique(valid)) == len(valid), "duplicate slots in one call"
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        b, pos = split_slot(int(slot), block_size)
        a = address(view, layer, b, pos)
        out[a:a + view.row_bytes] = rows[t]
    return out


def copy_blocks(image: np.ndarray, view: CacheView, pairs, num_layers: int, block_size: int) -> np.ndarray:
    """Copy-on-write's data movement: for each (src, dst) block pair and each layer, the dst page takes the
    src page's bytes.

    "vLLM 技术内幕", §2.2: a sequence about to write into a block whose reference count is above 1 gets
    a new physical block, the contents are copied, and the old block's count drops by one. The count
    and the allocation belong to the block manager; what reaches the device is the copy. A page is
    the block_size rows of one block in one layer of the view ("vLLM KV Cache Layout 可视化": rows of
    a block are contiguous, pos * row_bytes apart). Every copy reads the image as it was before the
    call; pairs whose pages overlap are a caller error (asserted here).
    """
    src_img = np.asarray(image, dtype=np.uint8)
    out = np.array(src_img, copy=True)
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    dsts = pairs[:, 1]
    assert len(np.unique(dsts)) == len(dsts), "two pairs write one block"
    assert not set(pairs[:, 0].tolist()) & set(dsts.tolist()), "a block is both copied and overwritten"
    page = block_size * view.row_bytes
    for s, d in pairs:
        for layer in range(num_layers):
            a_s = address(view, layer, int(s), 0)
            a_d = address(view, layer, int(d), 0)
            out[a_d:a_d + page] = src_img[a_s:a_s + page]
    return out

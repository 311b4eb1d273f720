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

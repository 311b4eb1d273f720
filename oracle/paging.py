"""Integer side of paging: blocks, slots, cache views and byte addresses.

Sources:
* "KV Cache 与推理服务内存管理", PagedAttention section: a prompt of n tokens
  takes ceil(n / BLOCK_SIZE) blocks at prefill. A decode token at position p
  sits in logical block p // BLOCK_SIZE at offset p % BLOCK_SIZE. The block
  table maps a logical block id to a physical block id.
* "deep dive into vLLM 05", §1.3: the 2050 / 2350-token block counts, and
  the rule that only full blocks go into the prefix cache.
* "vLLM KV Cache Layout 可视化":
  - terms section: slot, block, page = block_size x row width;
  - KVCacheTensor section: view {offset, layer_stride, block_stride} and the
    address formula;
  - layout section: stride rules of layer-outer and block-outer layouts;
  - slot_mapping section: slot = physical block x block_size + position;
  - kernel section: the slot is split back and multiplied by the strides.
"""

from __future__ import annotations

from dataclasses import dataclass


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """ceil(num_tokens / block_size): blocks a sequence of num_tokens occupies."""
    return -(-int(num_tokens) // int(block_size))


def full_blocks(num_tokens: int, block_size: int) -> int:
    """Blocks completely filled by num_tokens; only these can be shared as a cached prefix."""
    return int(num_tokens) // int(block_size)


def logical_block_and_offset(position: int, block_size: int):
    """Token position -> (logical block id, offset inside the block)."""
    return int(position) // int(block_size), int(position) % int(block_size)


def slot_of(table_row, position: int, block_size: int) -> int:
    """slot_mapping value of a token: physical block * block_size + in-block offset."""
    lb, off = logical_block_and_offset(position, block_size)
    return int(table_row[lb]) * int(block_size) + off


def split_slot(slot: int, block_size: int):
    """Inverse of slot_of as the write kernel does it: (block = slot / bs, position = slot % bs)."""
    return int(slot) // int(block_size), int(slot) % int(block_size)


@dataclass(frozen=True)
class CacheView:
    """One view over a flat cache allocation (the KVCacheTensor parameters plus row width)."""
    offset: int          # bytes to layer 0, block 0 of this view
    layer_stride: int    # bytes between the same block number of adjacent layers
    block_stride: int    # bytes between adjacent block numbers within a layer
    row_bytes: int       # bytes between adjacent tokens within a block (the row width)


def address(view: CacheView, layer: int, block: int, position: int) -> int:
    """Byte address = offset + layer*layer_stride + block*block_stride + position*row_bytes."""
    return (view.offset + int(layer) * view.layer_stride + int(block) * view.block_stride
            + int(position) * view.row_bytes)


def page_bytes(block_size: int, row_bytes: int) -> int:
    """A page is one block's worth of rows for one layer of one cache."""
    return int(block_size) * int(row_bytes)


def dense_row_bytes(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """Row width of a [num_blocks, block_size, num_kv_heads, head_dim] cache: one token, all heads."""
    return int(num_kv_heads) * int(head_dim) * int(elem_bytes)


def layer_outer_views(caches, block_size: int, num_blocks: int):
    """Views for an L-first layout (LBHNC / LBNHC).

    ``caches`` is a list of (name, row_bytes, num_layers). Each cache's layers
    are laid out one after another, and each layer covers all its blocks
    contiguously. So block_stride = page and layer_stride = page * num_blocks.
    Caches follow one another in list order.
    """
    views, base = {}, 0
    for name, row, nl in caches:
        page = page_bytes(block_size, row)
        views[name] = CacheView(offset=base, layer_stride=page * num_blocks, block_stride=page,
                                row_bytes=row)
        base += nl * page * num_blocks
    return views


def block_outer_views(caches, block_size: int):
    """Views for a B-first layout (BLHNC / BLNHC).

    One physical block holds the page of every layer of every cache, in list
    order. So layer_stride = page, and every view shares block_stride = the
    total bytes of one block. A view's offset is where its layer-0 page starts
    inside the block.
    """
    views, base = {}, 0
    pages = [(name, page_bytes(block_size, row), row, nl) for name, row, nl in caches]
    block_total = sum(p * nl for _, p, _, nl in pages)
    for name, page, row, nl in pages:
        views[name] = CacheView(offset=base, layer_stride=page, block_stride=block_total, row_bytes=row)
        base += nl * page
    return views, block_total

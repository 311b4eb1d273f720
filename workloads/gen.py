"""Seeded generators: context lengths, block tables, slot integers, values.

Structure (lengths, permutations) comes from NumPy PCG64. Bulk values come
from a torch generator seeded from the same workload seed. That torch
generator runs on the CPU for small pools and on the device for the
multi-gigabyte ones.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

INT32_PAD = np.iinfo(np.int32).max  # block-table padding past a sequence's last block

SEEDS = {"tiny": 1301, "mha13b": 1302, "gqa_prefix": 1303, "long_mixed": 1304, "dsa_mla": 1305}

WORKLOADS = {
    "tiny": dict(num_seqs=4, context_lens=[1, 17, 130, 300], num_q_heads=8, num_kv_heads=8,
                 head_dim=128, dtype="f16", block_size=16, num_blocks=64),
    "mha13b": dict(num_seqs=64, ctx_low=128, ctx_high=2048, num_q_heads=40, num_kv_heads=40,
                   head_dim=128, dtype="f16", block_size=16, num_blocks=12288),
    "gqa_prefix": dict(num_seqs=256, prefix_tokens=2000, suffix_median=300, suffix_sigma=1.0,
                       suffix_low=1, suffix_high=6000, num_q_heads=32, num_kv_heads=8,
                       head_dim=128, dtype="bf16", block_size=16),
    "long_mixed": dict(num_long=8, long_ctx=32768, partition_size=512, prompt_tokens=3000,
                       chunks=[2048, 952], decode_a_ctx=1000, decode_b_ctx=2000,
                       num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                       block_size=16, num_blocks=17408),
    "dsa_mla": dict(num_layers=2, block_size=64, num_blocks=9216, mla_row_bytes=656,
                    indexer_row_bytes=132, num_seqs=64, ctx_low=1024, ctx_high=8192,
                    num_q_heads=128, latent_dim=512, rope_dim=64, scale_group=128,
                    index_heads=64, index_dim=128, top_k=2048),
}


def workload(name: str) -> dict:
    d = dict(WORKLOADS[name])
    d["name"] = name
    d["seed"] = SEEDS[name]
    return d


# --------------------------------------------------------------------------
# Value draws (storage bits)
# --------------------------------------------------------------------------

def f16_nan_bits() -> int:
    return 0x7E00


def bf16_nan_bits() -> int:
    return 0x7FC0


def _torch():
    import torch  # imported lazily so that plain NumPy users do not pay for it
    return torch


def draw_bits(seed: int, shape, dtype: str, device: str = "cpu"):
    """N(0,1) float32 draws rounded (RNE) to fp16/bf16; returns a torch int16 tensor of bits.

    Large shapes are drawn in chunks to bound temporary float32 memory.
    """
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=tdt, device=device)
    chunk = 1 << 26
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = torch.randn(e - s, generator=g, device=device, dtype=torch.float32).to(tdt)
    return out.view(torch.int16).reshape(shape)


def draw_context_lens(rng: np.random.Generator, name: str, p: dict) -> np.ndarray:
    if name == "tiny":
        return np.asarray(p["context_lens"], dtype=np.int32)
    if name in ("mha13b", "dsa_mla"):
        return rng.integers(p["ctx_low"], p["ctx_high"] + 1, size=p["num_seqs"]).astype(np.int32)
    if name == "gqa_prefix":
        s = rng.lognormal(mean=math.log(p["suffix_median"]), sigma=p["suffix_sigma"], size=p["num_seqs"])
        s = np.clip(np.round(s), p["suffix_low"], p["suffix_high"]).astype(np.int32)
        return (p["prefix_tokens"] + s).astype(np.int32)
    raise KeyError(name)


# --------------------------------------------------------------------------
# Allocator / scheduler stand-ins (host control plane, outside the hot path)
# --------------------------------------------------------------------------

def allocate_block_tables(rng: np.random.Generator, context_lens, block_size: int, num_blocks: int,
                          width: int | None = None, shared_prefix_blocks: int = 0):
    """Give each sequence ceil(ctx / block_size) physical blocks from a seeded permutation.

    Blocks are handed out in sequence order from the permuted free list, as
    the allocator on the "KV Cache 与推理服务内存管理" page does at prefill.
    With ``shared_prefix_blocks = n``, the first n entries of every table are
    the same n physical blocks (a prompt shared with ref_cnt > 1, as on the
    "deep dive into vLLM 05" page, §3.1); only the remainder is private.
    Padding entries hold INT32_PAD. Returns (tables int32 [B, width], perm).
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    need = (ctx + block_size - 1) // block_size
    if width is None:
        width = max(1, int(need.max()))
    perm = rng.permutation(num_blocks).astype(np.int64)
    tables = np.full((len(ctx), width), INT32_PAD, dtype=np.int32)
    cursor = 0
    shared = perm[:shared_prefix_blocks]
    cursor += shared_prefix_blocks
    for b, n in enumerate(need):
        n = int(n)
        k = min(n, shared_prefix_blocks)
        tables[b, :k] = shared[:k]
        priv = n - k
        if cursor + priv > num_blocks:
            raise ValueError("block pool too small for the drawn contexts")
        tables[b, k:n] = perm[cursor:cursor + priv]
        cursor += priv
    return tables, perm


def slots_for_positions(table_row, positions, block_size: int) -> np.ndarray:
    """The scheduler's per-token integer: physical block * block_size + in-block position.

    This is the value the "vLLM KV Cache Layout 可视化" page calls
    slot_mapping (section on slot_mapping). The kernels undo it.
    """
    pos = np.asarray(positions, dtype=np.int64)
    row = np.asarray(table_row, dtype=np.int64)
    return row[pos // block_size] * block_size + pos % block_size


def used_blocks(tables: np.ndarray) -> np.ndarray:
    t = tables[tables != INT32_PAD]
    return np.unique(t.astype(np.int64))


# --------------------------------------------------------------------------
# Dense (fp16 / bf16, NHD rows) decode cases
# --------------------------------------------------------------------------

@dataclass
class DenseCase:
    name: str
    dtype: str
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    context_lens: np.ndarray           # int32 [B]
    block_tables: np.ndarray           # int32 [B, W]
    seed: int
    k_pool: object = None              # torch int16 [nb, bs, Hkv, D] bits
    v_pool: object = None
    q: object = None                   # torch int16 [B, Hq, D] bits
    new_k: object = None               # torch int16 [B, Hkv, D] bits: each sequence's last token
    new_v: object = None
    new_slots: np.ndarray | None = None  # int64 [B] slot of each sequence's last token
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(len(self.context_lens))

    @property
    def row_bytes(self) -> int:
        return self.num_kv_heads * self.head_dim * 2


def make_dense_case(name: str, device: str = "cpu", seed: int | None = None, context_lens=None,
                    num_blocks: int | None = None, num_q_heads: int | None = None,
                    num_kv_heads: int | None = None, block_size: int | None = None,
                    dtype: str | None = None, copied_prefix: bool = False, with_pools: bool = True,
                    head_dim: int | None = None) -> DenseCase:
    """Build one dense decode workload.

    ``context_lens``, ``num_blocks`` and the head counts override the named
    recipe (for small parity cases). For ``gqa_prefix``, ``copied_prefix=True``
    gives every sequence its own byte-identical copy of the 125 prompt blocks
    instead of sharing them.
    """
    p = workload(name)
    seed = p["seed"] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    bs = block_size or p["block_size"]
    dt = dtype or p["dtype"]
    hq = num_q_heads or p["num_q_heads"]
    hkv = num_kv_heads or p["num_kv_heads"]
    d = head_dim or p["head_dim"]
    ctx = (np.asarray(context_lens, dtype=np.int32) if context_lens is not None
           else draw_context_lens(rng, name, p))
    shared = 0
    if name == "gqa_prefix" and context_lens is None:
        shared = p["prefix_tokens"] // bs
    need = (ctx.astype(np.int64) + bs - 1) // bs
    if num_blocks is None:
        num_blocks = p.get("num_blocks")
        if num_blocks is None:  # size the pool to the need plus a little slack
            total = int(need.sum()) - (len(ctx) - 1) * shared if (shared and not copied_prefix) else int(need.sum())
            num_blocks = total + 64
    tables, _ = allocate_block_tables(rng, ctx, bs, num_blocks,
                                      shared_prefix_blocks=0 if copied_prefix else shared)
    case = DenseCase(name=name, dtype=dt, block_size=bs, num_blocks=int(num_blocks), num_q_heads=hq,
                     num_kv_heads=hkv, head_dim=d, scale=1.0 / math.sqrt(d), context_lens=ctx,
                     block_tables=tables, seed=seed)
    last = np.maximum(ctx.astype(np.int64) - 1, 0)
    case.new_slots = np.array([slots_for_positions(tables[b], [last[b]], bs)[0] if ctx[b] > 0 else -1
                               for b in range(len(ctx))], dtype=np.int64)
    case.extra["shared_prefix_blocks"] = shared
    case.extra["copied_prefix"] = copied_prefix
    if with_pools:
        fill_dense_values(case, device=device)
    return case


def fill_dense_values(case: DenseCase, device: str = "cpu") -> None:
    """Draw Q, the K/V pools and each sequence's new (last-token) K/V rows.

    Blocks that no table references are NaN-filled. For the copied-prefix
    variant the private prompt blocks are byte copies of one drawn prompt.
    """
    torch = _torch()
    s = case.seed
    shape = (case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim)
    case.k_pool = draw_bits(s * 16 + 1, shape, case.dtype, device)
    case.v_pool = draw_bits(s * 16 + 2, shape, case.dtype, device)
    case.q = draw_bits(s * 16 + 3, (case.num_seqs, case.num_q_heads, case.head_dim), case.dtype, device)
    case.new_k = draw_bits(s * 16 + 4, (case.num_seqs, case.num_kv_heads, case.head_dim), case.dtype, device)
    case.new_v = draw_bits(s * 16 + 5, (case.num_seqs, case.num_kv_heads, case.head_dim), case.dtype, device)
    nan = f16_nan_bits() if case.dtype == "f16" else bf16_nan_bits()
    used = used_blocks(case.block_tables)
    mask = np.ones(case.num_blocks, dtype=bool)
    mask[used] = False
    unused = torch.from_numpy(np.nonzero(mask)[0].astype(np.int64)).to(device)
    if unused.numel():
        case.k_pool.index_fill_(0, unused, nan)  # both NaN patterns fit in int16
        case.v_pool.index_fill_(0, unused, nan)
    if case.extra.get("copied_prefix"):
        # Same draw as the shared variant would see for its prompt blocks: copy
        # the first sequence's prompt blocks into every other sequence's.
        n = workload(case.name)["prefix_tokens"] // case.block_size
        src = torch.from_numpy(case.block_tables[0, :n].astype(np.int64)).to(device)
        for b in range(1, case.num_seqs):
            dst = torch.from_numpy(case.block_tables[b, :n].astype(np.int64)).to(device)
            case.k_pool.index_copy_(0, dst, case.k_pool.index_select(0, src))
            case.v_pool.index_copy_(0, dst, case.v_pool.index_select(0, src))


# --------------------------------------------------------------------------
# Mixed chunked-prefill + decode case
# --------------------------------------------------------------------------

@dataclass
class ChunkCase:
    """One varlen call: sequences with query counts and total lengths (current tokens included)."""
    dtype: str
    block_size: int
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    scale: float
    seq_lens: np.ndarray        # int32 [S]: tokens in cache for each sequence, this step's included
    query_lens: np.ndarray      # int32 [S]
    query_start_loc: np.ndarray  # int32 [S+1]
    block_tables: np.ndarray    # int32 [S, W]
    k_pool: object = None
    v_pool: object = None
    q: object = None            # torch int16 [total_q, Hq, D]
    seed: int = 0

    @property
    def total_q(self) -> int:
        return int(self.query_start_loc[-1])


def make_chunk_case(step: int = 1, device: str = "cpu", seed: int | None = None, seq_lens=None,
                    query_lens=None, num_blocks: int | None = None, num_q_heads: int | None = None,
                    num_kv_heads: int | None = None, dtype: str | None = None,
                    block_size: int | None = None, with_pools: bool = True,
                    tables_for_lens=None) -> ChunkCase:
    """The long-context mixed call, or a small varlen case when lengths are given.

    Default (the ``long_mixed`` recipe): 8 decodes at 32768 tokens, decodes A
    (1000) and B (2000), and the prompt chunk. ``step=1`` is the 2048-token
    chunk at total length 2048. ``step=2`` is the 952-token chunk at total
    3000, with every decode one token longer. Block tables are sized for the
    final lengths (``tables_for_lens``), so both steps share one pool and one
    table array.
    """
    p = workload("long_mixed")
    seed = p["seed"] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    bs = block_size or p["block_size"]
    if seq_lens is None:
        nl = p["num_long"]
        if step == 1:
            seq_lens = [p["long_ctx"]] * nl + [p["decode_a_ctx"], p["decode_b_ctx"], p["chunks"][0]]
            query_lens = [1] * (nl + 2) + [p["chunks"][0]]
        else:
            seq_lens = [p["long_ctx"] + 1] * nl + [p["decode_a_ctx"] + 1, p["decode_b_ctx"] + 1,
                                                   p["prompt_tokens"]]
            query_lens = [1] * (nl + 2) + [p["chunks"][1]]
        tables_for_lens = ([p["long_ctx"] + 1] * nl + [p["decode_a_ctx"] + 1, p["decode_b_ctx"] + 1,
                                                       p["prompt_tokens"]])
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    if tables_for_lens is None:
        tables_for_lens = seq_lens
    nb = num_blocks or p["num_blocks"]
    tables, _ = allocate_block_tables(rng, tables_for_lens, bs, nb)
    qsl = np.zeros(len(seq_lens) + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(query_lens)
    hq = num_q_heads or p["num_q_heads"]
    hkv = num_kv_heads or p["num_kv_heads"]
    d = p["head_dim"]
    case = ChunkCase(dtype=dtype or p["dtype"], block_size=bs, num_blocks=int(nb), num_q_heads=hq,
                     num_kv_heads=hkv, head_dim=d, scale=1.0 / math.sqrt(d), seq_lens=seq_lens,
                     query_lens=query_lens, query_start_loc=qsl, block_tables=tables, seed=seed)
    if with_pools:
        shape = (case.num_blocks, bs, hkv, d)
        case.k_pool = draw_bits(seed * 16 + 1, shape, case.dtype, device)
        case.v_pool = draw_bits(seed * 16 + 2, shape, case.dtype, device)
        case.q = draw_bits(seed * 16 + 3 + step, (case.total_q, hq, d), case.dtype, device)
    return case


# --------------------------------------------------------------------------
# DSA dual cache: packed MLA and indexer rows
# --------------------------------------------------------------------------

def draw_mla_rows(seed: int, n: int, device: str = "cpu"):
    """Packed 656-byte MLA rows as a torch uint8 tensor [n, 656].

    Bytes [0, 512) hold 512 e4m3 latent values. Bytes [512, 528) hold 4
    little-endian float32 scales, scale k covering latent values
    [128k, 128k + 128). Bytes [528, 656) hold 64 little-endian bf16 RoPE values.
    The latent values are x / scale rounded to float8_e4m3fn by torch's cast,
    where x ~ N(0, 1) and scale = amax / 448 over each 128-group.
    """
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(n, 4, 128, generator=g, device=device, dtype=torch.float32)
    amax = x.abs().amax(dim=2, keepdim=True).clamp_min(1e-30)
    scale = (amax / 448.0).to(torch.float32)
    lat = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, 512)
    rope = torch.randn(n, 64, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    rows = torch.empty(n, 656, dtype=torch.uint8, device=device)
    rows[:, :512] = lat
    rows[:, 512:528] = scale.reshape(n, 4).contiguous().view(torch.uint8)
    rows[:, 528:656] = rope.contiguous().view(torch.uint8)
    return rows


def draw_indexer_rows(seed: int, n: int, device: str = "cpu"):
    """Packed 132-byte indexer rows [n, 132]: 128 e4m3 key values, then one float32 scale."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(n, 128, generator=g, device=device, dtype=torch.float32)
    scale = (x.abs().amax(dim=1, keepdim=True).clamp_min(1e-30) / 448.0).to(torch.float32)
    key = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8)
    rows = torch.empty(n, 132, dtype=torch.uint8, device=device)
    rows[:, :128] = key
    rows[:, 128:132] = scale.contiguous().view(torch.uint8)
    return rows


def draw_index_queries(seed: int, num_seqs: int, num_heads: int, device: str = "cpu"):
    """Lightning-indexer inputs of num_seqs decode tokens: queries as bf16 bits (torch int16
    [B, H, 128], N(0, 1)) and head weights (torch float32 [B, H], N(0, 1 / H))."""
    torch = _torch()
    q = draw_bits(seed, (num_seqs, num_heads, 128), "bf16", device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 1)
    w = torch.randn(num_seqs, num_heads, generator=g, device=device, dtype=torch.float32) / math.sqrt(num_heads)
    return q, w


@dataclass
class MlaCase:
    num_layers: int
    block_size: int
    num_blocks: int
    block_bytes: int
    num_q_heads: int
    scale: float
    context_lens: np.ndarray        # int32 [B]
    block_tables: np.ndarray        # int32 [B, W]
    populate_slots: np.ndarray      # int64 [N]: positions 0 .. ctx-2 of every sequence
    step_slots: np.ndarray          # int64 [B]: position ctx-1 of every sequence
    seed: int
    q: object = None                # torch int16 [B, Hq, 576] bf16 bits
    mla_rows: list = field(default_factory=list)      # per layer: uint8 [N, 656]
    idx_rows: list = field(default_factory=list)      # per layer: uint8 [N, 132]
    step_mla_rows: list = field(default_factory=list)  # per layer: uint8 [B, 656]
    step_idx_rows: list = field(default_factory=list)  # per layer: uint8 [B, 132]
    index_heads: int = 64
    top_k: int = 2048
    q_index: object = None          # torch int16 [B, index_heads, 128] bf16 bits
    index_weights: object = None    # torch float32 [B, index_heads]


def make_mla_case(device: str = "cpu", seed: int | None = None, context_lens=None,
                  num_blocks: int | None = None, num_q_heads: int | None = None,
                  with_rows: bool = True, block_size: int | None = None) -> MlaCase:
    p = workload("dsa_mla")
    seed = p["seed"] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    bs = block_size or p["block_size"]
    ctx = (np.asarray(context_lens, dtype=np.int32) if context_lens is not None
           else draw_context_lens(rng, "dsa_mla", p))
    nb = num_blocks or p["num_blocks"]
    tables, _ = allocate_block_tables(rng, ctx, bs, nb)
    pop, step = [], []
    for b, c in enumerate(ctx):
        c = int(c)
        if c > 1:
            pop.append(slots_for_positions(tables[b], np.arange(c - 1), bs))
        step.append(slots_for_positions(tables[b], [max(c - 1, 0)], bs)[0] if c > 0 else -1)
    pop = np.concatenate(pop) if pop else np.zeros(0, dtype=np.int64)
    page_mla, page_idx = bs * p["mla_row_bytes"], bs * p["indexer_row_bytes"]
    hq = num_q_heads or p["num_q_heads"]
    case = MlaCase(num_layers=p["num_layers"], block_size=bs, num_blocks=int(nb),
                   block_bytes=p["num_layers"] * (page_mla + page_idx), num_q_heads=hq,
                   scale=1.0 / math.sqrt(p["latent_dim"] + p["rope_dim"]), context_lens=ctx,
                   block_tables=tables, populate_slots=pop.astype(np.int64),
                   step_slots=np.asarray(step, dtype=np.int64), seed=seed)
    if with_rows:
        B = len(ctx)
        case.q = draw_bits(seed * 16 + 3, (B, hq, p["latent_dim"] + p["rope_dim"]), "bf16", device)
        for layer in range(case.num_layers):
            case.mla_rows.append(draw_mla_rows(seed * 16 + 5 + 4 * layer, len(pop), device))
            case.idx_rows.append(draw_indexer_rows(seed * 16 + 6 + 4 * layer, len(pop), device))
            case.step_mla_rows.append(draw_mla_rows(seed * 16 + 7 + 4 * layer, B, device))
            case.step_idx_rows.append(draw_indexer_rows(seed * 16 + 8 + 4 * layer, B, device))
        case.index_heads, case.top_k = p["index_heads"], p["top_k"]
        case.q_index, case.index_weights = draw_index_queries(seed * 16 + 13, B, p["index_heads"], device)
    return case

"""GPU parity of pa_copy_blocks (copy-on-write's data movement) against oracle.cache_write.copy_blocks.

Caches of 3 layers in the layer-outer and block-outer layouts of "vLLM KV Cache Layout 可视化" (K and
V views, 16-byte and 4-byte rows) get random disjoint (src, dst) pairs, plus pairs with ids outside
the pool, which are skipped; every byte must match the oracle. Then copy-on-write itself ("vLLM 技术
内幕" §2.2): sequences that share a prompt's blocks get private copies through pa_copy_blocks, and
decode through the private tables is bitwise equal to decode through the shared ones.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_130_amd as pa
from oracle import cache_write as W
from oracle import paging as P
from helpers import image_of

pytestmark = pytest.mark.gpu

L = 3


def views(layout, row, bs, nb):
    if layout == "layer":
        return P.CacheView(0, nb * bs * row, bs * row, row), L * nb * bs * row
    return P.CacheView(0, bs * row, L * bs * row, row), nb * L * bs * row


def to_pa(v):
    return pa.CacheView(v.offset, v.layer_stride, v.block_stride, v.row_bytes)


@pytest.mark.parametrize("layout", ["layer", "block"])
@pytest.mark.parametrize("row_k,row_v,bs", [(2048, 2048, 16), (656, 132, 64), (256, 0, 32)])
@pytest.mark.parametrize("npairs", [1, 7, 300])
def test_copy_blocks_matches_oracle(layout, row_k, row_v, bs, npairs):
    rng = np.random.default_rng(npairs + row_k + bs)
    nb = 2 * npairs + 8
    kv, kbytes = views(layout, row_k, bs, nb)
    kimg = torch.from_numpy(rng.integers(0, 256, kbytes, dtype=np.uint8)).cuda()
    vimg = None
    if row_v:
        vv, vbytes = views(layout, row_v, bs, nb)
        vimg = torch.from_numpy(rng.integers(0, 256, vbytes, dtype=np.uint8)).cuda()
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:npairs], perm[npairs:2 * npairs]], axis=1).astype(np.int64)
    bad = np.array([[nb, perm[-1]], [perm[-2], -1]], dtype=np.int64)   # skipped: ids outside the pool
    all_pairs = np.concatenate([pairs, bad]) if npairs > 1 else pairs
    k_before, v_before = image_of(kimg), image_of(vimg) if row_v else None
    pa.pa_copy_blocks(torch.from_numpy(all_pairs).cuda(), kimg, to_pa(kv), L, bs, nb,
                      v_cache=vimg, v_view=to_pa(vv) if row_v else None)
    torch.cuda.synchronize()
    assert np.array_equal(image_of(kimg), W.copy_blocks(k_before, kv, pairs, L, bs))
    if row_v:
        assert np.array_equal(image_of(vimg), W.copy_blocks(v_before, vv, pairs, L, bs))


def test_copy_on_write_of_a_shared_prompt_keeps_decode_bitwise():
    rng = np.random.default_rng(42)
    bs, nb, hq, hkv, d = 16, 64, 32, 8, 128
    row = hkv * d * 2
    kd = torch.randn(nb, bs, hkv, d, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).cuda()
    vd = torch.randn(nb, bs, hkv, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).cuda()
    prompt = [5, 9, 2, 30, 11]              # 5 blocks of prompt, shared by 3 sequences
    tails = [[40], [41, 42], [43]]
    ctx = [5 * bs + 7, 5 * bs + 20, 5 * bs + 1]
    shared = np.full((3, 8), np.iinfo(np.int32).max, dtype=np.int32)
    for b in range(3):
        ids = prompt + tails[b]
        shared[b, :len(ids)] = ids
    # Copy-on-write for sequences 1 and 2: private copies of the prompt blocks.
    fresh = [[50, 51, 52, 53, 54], [55, 56, 57, 58, 59]]
    pairs = np.array([[s, f] for fb in fresh for s, f in zip(prompt, fb)], dtype=np.int64)
    view = pa.dense_view(bs, hkv, d)
    pa.pa_copy_blocks(torch.from_numpy(pairs).cuda(), kd, view, 1, bs, nb, v_cache=vd, v_view=view)
    private = shared.copy()
    private[1, :5] = fresh[0]
    private[2, :5] = fresh[1]
    q = torch.randn(3, hq, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    desc = pa.dense_desc("bf16", hq, hkv, d, bs, nb, kd.numel() * 2, vd.numel() * 2, 32)
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, 3, max(ctx))), dtype=torch.uint8, device="cuda")
    outs = []
    for tables in (shared, private):
        out = torch.empty(3, hq, d, dtype=torch.int16, device="cuda")
        pa.pa_decode(out, q.view(torch.int16), kd, vd, torch.from_numpy(tables).cuda(),
                     torch.tensor(ctx, dtype=torch.int32).cuda(), max(ctx), d ** -0.5, desc, ws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    assert row == kd[0, 0].numel() * 2

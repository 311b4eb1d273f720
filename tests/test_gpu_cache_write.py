"""GPU parity of pa_reshape_and_cache on its own: every byte of the cache image, sentinels included.

Row widths cover the dense rows of the workloads (one 128-dim head, 8 and 40 heads of 128 at 16
bits), the DSA rows (656 B, 16-byte copies; 132 B, 4-byte copies) and a short 20-byte row. Token
counts cover partial waves and work-groups; slots include padding (-1), one past the pool and
shuffled positions; sources have a pitch wider than the row; two views share one slot_mapping with
different layers' offsets. The oracle is oracle.cache_write ("vLLM KV Cache Layout 可视化", kernel
section: block = slot / block_size, position = slot % block_size).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_130_amd as pa
from oracle import cache_write as W
from oracle import paging as P
from helpers import image_of

pytestmark = pytest.mark.gpu


def run(row_k, row_v, T, bs, nb, layer, seed, pitch_pad=0):
    rng = np.random.default_rng(seed)
    # Layer-outer views of a 2-layer allocation per cache.
    kview = P.CacheView(0, nb * bs * row_k, bs * row_k, row_k)
    vview = P.CacheView(0, nb * bs * row_v, bs * row_v, row_v) if row_v else None
    kimg = torch.full((2 * nb * bs * row_k,), 0xA5, dtype=torch.uint8, device="cuda")
    vimg = torch.full((2 * nb * bs * row_v,), 0x5A, dtype=torch.uint8, device="cuda") if row_v else None
    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    slots[rng.random(T) < 0.2] = -1
    if T > 3:
        slots[3] = nb * bs          # one past the pool: skipped
    ksrc = torch.from_numpy(rng.integers(0, 256, (T, row_k + pitch_pad), dtype=np.uint8)).cuda()
    vsrc = torch.from_numpy(rng.integers(0, 256, (T, row_v + pitch_pad), dtype=np.uint8)).cuda() if row_v else None
    to_pa = lambda v: pa.CacheView(v.offset, v.layer_stride, v.block_stride, v.row_bytes)
    pa.pa_reshape_and_cache(ksrc, torch.from_numpy(slots).cuda(), kimg, to_pa(kview), layer, bs, nb,
                            v=vsrc, v_cache=vimg, v_view=to_pa(vview) if row_v else None)
    torch.cuda.synchronize()
    ok = slots.copy()
    ok[ok >= nb * bs] = -1          # the oracle asserts in-range slots; out-of-range ones are not written
    kwant = W.reshape_and_cache(np.full(kimg.numel(), 0xA5, dtype=np.uint8),
                                ksrc.cpu().numpy()[:, :row_k], ok, kview, layer, bs)
    assert np.array_equal(image_of(kimg), kwant)
    if row_v:
        vwant = W.reshape_and_cache(np.full(vimg.numel(), 0x5A, dtype=np.uint8),
                                    vsrc.cpu().numpy()[:, :row_v], ok, vview, layer, bs)
        assert np.array_equal(image_of(vimg), vwant)


@pytest.mark.parametrize("row_k,row_v", [(256, 256), (2048, 2048), (10240, 10240), (656, 132), (20, 0)])
@pytest.mark.parametrize("T", [1, 5, 17, 1000])
def test_cache_write_matches_oracle(row_k, row_v, T):
    bs, nb = 16, max(8, (T + 15) // 16 + 4)
    run(row_k, row_v, T, bs, nb, layer=T % 2, seed=row_k + T)


def test_cache_write_with_wide_source_pitch():
    run(2048, 2048, 300, 64, 8, layer=1, seed=3, pitch_pad=48)

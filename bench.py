"""Benchmark of the paged-KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra] [--no-cpu-baseline]

The JSON line is for the 13B-shaped MHA decode (64 sequences, contexts U[128, 2048], 40 heads of
128, fp16, block size 16). One step writes each sequence's new K/V row through slot_mapping
(pa_reshape_and_cache), then attends every sequence to its whole paged context (pa_decode). Inputs are
seeded synthetic draws resident in HBM when timing starts.

Timing: every timed call (or step) is preceded, outside its HIP events, by a write of a 512 MiB
device buffer and a read of a second one (see Flush), which evicts the 256 MB Infinity Cache and the
L2s, so no call reads K/V left in a cache by the previous one. Events are recorded on the launch stream. Call-level figures are the
median (with p10/p90 and the mean) of at least 50 calls; the same figures without the flush sit
beside them as `*_warm`.

`value` is the step's algorithmic bytes per second over the mean flushed step time; decode tokens/s
sits beside it. `roofline` covers the pa_decode call (the dominant kernel): its algorithmic bytes over
its mean flushed duration. Its `traffic` is the HBM bytes per call from the committed rocprofv3
FETCH_SIZE/WRITE_SIZE runs (profiles/counters.json), given only when those runs were taken on the
kernel sources of this tree (`traffic_source` says which). `cpu_baseline` times the NumPy oracle on
the host cores over a bounded sample of the same batch, with all BLAS threads and again with one.
`extra` holds the other workloads, measured the same way: GQA-8 with a shared or copied 2000-token
prompt, long-context decode, FP8 caches, the mixed chunked-prefill steps, the DSA dual-cache writes
plus MLA decode, and the DSA sparse step (indexer scores, top-k, MLA decode over the selected slots).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

# Threads of the oracle's NumPy/BLAS (the CPU baseline), fixed before NumPy is first imported: the
# host's CPU share if the environment names one, else every core this process may run on.
_CPU_THREADS = os.environ.get("OMP_NUM_THREADS") or str(len(os.sched_getaffinity(0)))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, _CPU_THREADS)

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FLUSH_BYTES = 512 << 20     # written between timed calls: twice the 256 MB Infinity Cache
MIN_CALLS = 50              # calls behind every call-level median

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E peak, GB/s
FP8_SCALE = 2.0 ** -5       # K and V scale of the FP8 cache variants (N(0,1) values use codes up to ~160)
MFMA_BF16_PEAK_TF = 2500.0  # MI355X dense bf16/fp16 MFMA peak, TFLOP/s
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
KERNEL_SOURCES = ("api.hip", "cache_write.hip", "decode_dense.hip", "decode_fp8.hip", "decode_mfma.hip", "decode_mla.hip",
                  "dsa_indexer.hip", "prefill_mfma.hip", "decode_common.h", "decode_mfma.h",
                  "decode_mla.h", "mfma_common.h", "pa_device.h", "pa_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_130_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mha13b",
                    choices=["mha13b", "gqa_prefix", "gqa_prefix_copied", "long_decode", "long_mixed", "dsa_mla",
                             "mha13b_fp8", "gqa_prefix_copied_fp8", "prefill_chunk_2048", "prefill_chunk_952"])
    ap.add_argument("--partition", type=int, default=0, help="pa_decode partition_size (0: library choice)")
    ap.add_argument("--flush", default="write+read", choices=["write+read", "write"],
                    help="cache flush before each timed call: 512 MiB write then 512 MiB read, or the write alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the short runs of the other workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


class Flush:
    """Evicts the Infinity Cache and the L2s before a timed call (on the current stream).

    It writes a 512 MiB buffer, then reads a second one of 512 MiB. The write alone would leave up
    to 256 MB of its own dirty lines in the caches, and their write-back would then be charged to
    the timed call (measured: about 80 us more per call for the kernels whose K loads allocate in
    the cache, none for the fully nontemporal one). After the read, the caches hold only clean lines
    of the second buffer, so the call reads all of its K/V from HBM and writes nothing back for the
    flush. `mode="write"` keeps the write alone."""

    def __init__(self, torch, mode="write+read"):
        self.buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.rd = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if mode == "write+read" else None
        self.n = 0

    def __call__(self):
        self.n += 1
        self.buf.fill_(self.n & 0xFF)
        if self.rd is not None:
            self.sink = self.rd.sum()


def time_calls(torch, fn, n, flush=None):
    """Durations (ms) of n calls of fn, each between two HIP events on the current stream; `flush`
    runs before each call, outside the events."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in ev:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def dist(ms):
    """Median, mean, p10 and p90 of per-call durations (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": float(np.median(a)), "mean": float(a.mean()), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "calls": int(a.size)}


def call_stats(torch, fn, flush, calls=MIN_CALLS, warmup=3):
    """Flushed and warm distributions of one call."""
    for _ in range(warmup):
        fn()
    return dist(time_calls(torch, fn, calls, flush)), dist(time_calls(torch, fn, calls))


def traffic_for(name):
    """HBM bytes per call from the committed counter runs, and where they come from.

    The figure is given only if the runs were taken on the kernel sources of this tree (the hash of
    csrc/ recorded with them matches); it was not measured in this run."""
    if not os.path.exists(COUNTERS):
        return None, "no counter runs committed"
    with open(COUNTERS) as f:
        cnt = json.load(f)
    e = cnt.get(name)
    h = kernel_source_hash()
    if e and e.get("kernel_hash") == h:
        return e.get("hbm_bytes_per_call"), (f"profiles/counters.json: rocprofv3 FETCH_SIZE x {cnt['fetch_scale']:.3f} "
                                             f"+ WRITE_SIZE x {cnt['write_scale']:.3f} per dispatch, taken on kernel "
                                             f"sources {h} (not measured in this run)")
    return None, f"no counter run on kernel sources {h}"


# --------------------------------------------------------------------------
# Dense decode workloads
# --------------------------------------------------------------------------

def dense_case(name):
    import workloads
    if name == "mha13b":
        return workloads.make_dense_case("mha13b", device="cuda"), (
            "13B-shaped MHA decode: 64 seqs, ctx U[128,2048], 40/40 heads x 128, fp16, bs 16, 12288 blocks")
    if name in ("gqa_prefix", "gqa_prefix_copied"):
        copied = name.endswith("copied")
        return workloads.make_dense_case("gqa_prefix", device="cuda", copied_prefix=copied), (
            "GQA-8 decode: 256 seqs, shared 2000-token prompt (125 blocks) + lognormal suffix (median 300), "
            "32/8 heads x 128, bf16, bs 16" + ("; prompt blocks copied per sequence" if copied else ""))
    return workloads.make_dense_case("tiny", seed=1304, context_lens=[32768] * 8, num_blocks=17408, num_q_heads=32,
                                     num_kv_heads=8, dtype="bf16", device="cuda"), (
        "long-context decode: 8 seqs x 32768 tokens, 32/8 heads x 128, bf16, bs 16, partitions of 512")


def dense_bytes(case, row=None):
    """Algorithmic bytes: distinct K/V rows read once, Q, output, table entries, lengths; and the step's write."""
    import numpy as np
    ctx = case.context_lens.astype(np.int64)
    row = row or case.row_bytes
    B, Hq = case.num_seqs, case.num_q_heads
    if case.extra.get("shared_prefix_blocks") and not case.extra.get("copied_prefix"):
        unique_tokens = int(ctx.sum() - (B - 1) * case.extra["shared_prefix_blocks"] * case.block_size)
    else:
        unique_tokens = int(ctx.sum())
    nblk = int(((ctx + case.block_size - 1) // case.block_size).sum())
    fixed = B * Hq * case.head_dim * 2 * 2 + nblk * 4 + B * 4
    return int(ctx.sum()) * 2 * row + fixed, unique_tokens * 2 * row + fixed, B * 2 * row * 2 + B * 8


def run_dense(name, steps, warmup, partition, flush):
    import numpy as np
    import torch
    import paged_kv_cache_130_amd as pa
    fp8 = name.endswith("_fp8")
    case, wdesc = dense_case(name[:-4] if fp8 else name)
    B, Hq, D = case.num_seqs, case.num_q_heads, case.head_dim
    kd, vd = case.k_pool, case.v_pool
    view = pa.dense_view(case.block_size, case.num_kv_heads, D)
    part = partition or (512 if name == "long_decode" else 0)
    desc = pa.dense_desc(case.dtype, Hq, case.num_kv_heads, D, case.block_size, case.num_blocks, kd.numel() * 2,
                         vd.numel() * 2, part)
    row8 = None
    quant = {}
    if fp8:
        # The same workload with its K/V cache in FP8 (E4M3, one scale per cache): the 16-bit pools are
        # quantized on the device through pa_quantize_and_cache (every slot), queries become bf16.
        nb, bs, hkv = case.num_blocks, case.block_size, case.num_kv_heads
        tdt = torch.float16 if case.dtype == "f16" else torch.bfloat16
        row8 = hkv * D
        view8 = pa.dense_view(bs, hkv, D, 1)
        k8 = torch.empty((nb, bs, hkv, D), dtype=torch.uint8, device="cuda")
        v8 = torch.empty_like(k8)
        all_slots = torch.arange(nb * bs, dtype=torch.int64, device="cuda")
        ksrc = torch.nan_to_num(kd.view(tdt), nan=0.0).reshape(nb * bs, row8)
        vsrc = torch.nan_to_num(vd.view(tdt), nan=0.0).reshape(nb * bs, row8)

        def quantize_pool():
            pa.pa_quantize_and_cache(ksrc, all_slots, k8, view8, 0, bs, nb, FP8_SCALE,
                                     src_dtype="f16" if case.dtype == "f16" else "bf16", v=vsrc, v_cache=v8,
                                     v_view=view8, v_scale=FP8_SCALE)
        quantize_pool()
        qms = dist(time_calls(torch, quantize_pool, 5, flush))
        qbytes = 2 * nb * bs * row8 * 3 + nb * bs * 8
        quant = {"quantize_pool_ms": qms["median"], "quantize_pool_gbs": qbytes / (qms["median"] / 1e3) / 1e9}
        del ksrc, vsrc
        case.k_pool = case.v_pool = None
        kd, vd = k8, v8
        torch.cuda.empty_cache()
        case.q = case.q.view(tdt).to(torch.bfloat16).view(torch.int16)
        new_k = case.new_k.view(tdt).to(torch.bfloat16).reshape(B, row8)
        new_v = case.new_v.view(tdt).to(torch.bfloat16).reshape(B, row8)
        view = view8
        desc = pa.dense_desc("fp8", Hq, hkv, D, bs, nb, k8.numel(), v8.numel(), part, k_scale=FP8_SCALE,
                             v_scale=FP8_SCALE)
        wdesc += "; K/V cache in FP8 E4M3 (one scale per cache), bf16 queries"
    max_ctx = int(case.context_lens.max())
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, B, max_ctx)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, D, dtype=torch.int16, device="cuda")
    tables = torch.from_numpy(case.block_tables).cuda()
    lens = torch.from_numpy(case.context_lens).cuda()
    slots = torch.from_numpy(case.new_slots).cuda()
    stream = torch.cuda.current_stream()

    def write():
        if fp8:
            pa.pa_quantize_and_cache(new_k, slots, kd, view, 0, case.block_size, case.num_blocks, FP8_SCALE, v=new_v,
                                     v_cache=vd, v_view=view, v_scale=FP8_SCALE)
        else:
            pa.pa_reshape_and_cache(case.new_k, slots, kd, view, 0, case.block_size, case.num_blocks, v=case.new_v,
                                    v_cache=vd, v_view=view)

    def decode():
        pa.pa_decode(out, case.q, kd, vd, tables, lens, max_ctx, case.scale, desc, ws)

    for _ in range(warmup):
        write()
        decode()
    # The timed steps: flush, then write + decode between one pair of events (the decode alone is
    # timed by call_stats below).
    ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        ev_step[i][0].record(stream)
        write()
        decode()
        ev_step[i][1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    step_ms = float(np.mean([a.elapsed_time(b) for a, b in ev_step]))
    # Call-level distributions of the decode alone.
    flushed, warm = call_stats(torch, decode, flush, max(MIN_CALLS, steps))
    logical, unique, write_bytes = dense_bytes(case, row8)
    achieved = unique / (flushed["mean"] / 1e3) / 1e9
    traffic, traffic_src = traffic_for(name)
    cow = {}
    if name == "gqa_prefix_copied":
        # Copy-on-write of the shared prompt: every sequence's private prompt blocks take sequence 0's
        # prompt pages (the copies hold the same bytes, so the workload is unchanged).
        nprompt = case.extra["shared_prefix_blocks"]
        bt = case.block_tables
        pairs = np.array([[bt[0, j], bt[b, j]] for b in range(1, B) for j in range(nprompt)], dtype=np.int64)
        pairs_d = torch.from_numpy(pairs).cuda()
        cms = dist(time_calls(torch, lambda: pa.pa_copy_blocks(pairs_d, kd, view, 1, case.block_size, case.num_blocks,
                                                               v_cache=vd, v_view=view), 5, flush))
        cbytes = len(pairs) * 2 * 2 * case.block_size * case.row_bytes + pairs.nbytes
        cow = {"copy_on_write_pairs": len(pairs), "copy_on_write_ms": cms["median"],
               "copy_on_write_gbs": cbytes / (cms["median"] / 1e3) / 1e9}
    kernel = "decode_mfma_kernel" if (D == 128 and Hq // case.num_kv_heads >= 2) else "decode_dense_kernel"
    if fp8 and kernel == "decode_dense_kernel":
        kernel = "decode_fp8_kernel"
    return case, {
        "workload": wdesc,
        "ms_per_step": step_ms,
        "wall_ms_per_step_incl_flush": wall_ms,
        "value": (unique + write_bytes) / (step_ms / 1e3) / 1e9,
        "decode_tokens_per_s": B / (step_ms / 1e3),
        "decode_call_ms": flushed["median"],
        "decode_call_ms_mean": flushed["mean"],
        "decode_call_ms_p10_p90": [flushed["p10"], flushed["p90"]],
        "decode_call_calls": flushed["calls"],
        "decode_call_ms_warm": warm["median"],
        "decode_kv_gbs_unique": achieved,
        "decode_kv_gbs_logical": logical / (flushed["mean"] / 1e3) / 1e9,
        "decode_kv_gbs_counter": None if traffic is None else traffic / (flushed["mean"] / 1e3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "traffic_source": traffic_src,
                     "kernel": f"pa_decode ({kernel} + decode_reduce_kernel)", "algorithmic_bytes_per_call": unique,
                     "duration": "mean of the flushed calls"},
        "dtype": "fp8-e4m3 K/V, bf16 q" if fp8 else case.dtype,
        **cow,
        **quant,
        "config": {"num_seqs": B, "num_q_heads": Hq, "num_kv_heads": case.num_kv_heads, "head_dim": D,
                   "block_size": case.block_size, "num_blocks": case.num_blocks,
                   "sum_context_tokens": int(case.context_lens.sum()), "partition_size": part or "auto"},
    }


# --------------------------------------------------------------------------
# Mixed chunked prefill + decodes
# --------------------------------------------------------------------------

def chunk_flops(case):
    """2 * 2 * D * (visible tokens) summed over the chunk rows and query heads (QK and PV)."""
    total = 0
    for s in range(len(case.seq_lens)):
        n, ql = int(case.seq_lens[s]), int(case.query_lens[s])
        if ql < 2:
            continue
        first = n - ql
        total += sum(first + i + 1 for i in range(ql))
    return 4 * case.head_dim * case.num_q_heads * total


def chunk_alone(case, desc, ws, out, calls, warmup, flush):
    """The prompt chunk's rows alone (the same sequence and cache, no decode rows in the call): the
    prefill kernel's own MFMA rate."""
    import numpy as np
    import torch
    import paged_kv_cache_130_amd as pa
    c = len(case.seq_lens) - 1                     # the chunked prompt is the last sequence
    q0, q1 = int(case.query_start_loc[c]), int(case.query_start_loc[c + 1])
    only = [out[q0:q1], case.q[q0:q1], case.k_pool, case.v_pool,
            torch.from_numpy(np.ascontiguousarray(case.block_tables[c:c + 1])).cuda(),
            torch.from_numpy(case.seq_lens[c:c + 1].copy()).cuda(),
            torch.tensor([0, q1 - q0], dtype=torch.int32, device="cuda"), q1 - q0, int(case.seq_lens[c]),
            case.scale, desc, ws]
    cf, _ = call_stats(torch, lambda: pa.pa_prefill_chunk(*only), flush, calls, warmup)
    fl = chunk_flops(case)
    tf = fl / (cf["median"] / 1e3) / 1e12
    return {"chunk_alone_ms": cf["median"], "chunk_alone_ms_p10_p90": [cf["p10"], cf["p90"]],
            "chunk_alone_tflops": tf, "chunk_alone_mfma_frac": tf / MFMA_BF16_PEAK_TF}


def run_chunk_only(step, calls, warmup, flush):
    """One prompt chunk of the long-context mixed call, run alone (2048 tokens at total 2048, or 952
    at total 3000)."""
    import torch
    import paged_kv_cache_130_amd as pa
    import workloads
    case = workloads.make_chunk_case(step=step, device="cuda")
    desc = pa.dense_desc("bf16", case.num_q_heads, case.num_kv_heads, 128, 16, case.num_blocks,
                         case.k_pool.numel() * 2, case.v_pool.numel() * 2, 512)
    out = torch.empty(case.total_q, case.num_q_heads, 128, dtype=torch.int16, device="cuda")
    qlen, n = int(case.query_lens[-1]), int(case.seq_lens[-1])
    ws = torch.empty(max(16, pa.pa_prefill_workspace_bytes(desc, 1, qlen, qlen, n)), dtype=torch.uint8, device="cuda")
    r = chunk_alone(case, desc, ws, out, calls, warmup, flush)
    r["chunk_tokens"] = int(case.query_lens[-1])
    r["chunk_gflop"] = chunk_flops(case) / 1e9
    r["workload"] = (f"prompt chunk of {r['chunk_tokens']} tokens at total length {int(case.seq_lens[-1])}, causal over "
                     "paged context, 32/8 heads x 128, bf16, bs 16 (no decode rows)")
    return r


def run_mixed(calls, warmup, flush):
    import numpy as np
    import torch
    import paged_kv_cache_130_amd as pa
    import workloads
    res = {}
    for st in (1, 2):
        case = workloads.make_chunk_case(step=st, device="cuda")
        desc = pa.dense_desc("bf16", case.num_q_heads, case.num_kv_heads, 128, 16, case.num_blocks,
                             case.k_pool.numel() * 2, case.v_pool.numel() * 2, 512)
        S = len(case.seq_lens)
        max_q, max_s = int(case.query_lens.max()), int(case.seq_lens.max())
        ws = torch.empty(max(16, pa.pa_prefill_workspace_bytes(desc, S, case.total_q, max_q, max_s)),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty(case.total_q, case.num_q_heads, 128, dtype=torch.int16, device="cuda")
        args = [out, case.q, case.k_pool, case.v_pool, torch.from_numpy(case.block_tables).cuda(),
                torch.from_numpy(case.seq_lens).cuda(), torch.from_numpy(case.query_start_loc).cuda(), max_q, max_s,
                case.scale, desc, ws]
        flushed, warm = call_stats(torch, lambda: pa.pa_prefill_chunk(*args), flush, calls, warmup)
        ms = flushed["median"]
        dec_tokens = int(sum(int(n) for n, q in zip(case.seq_lens, case.query_lens) if q == 1))
        row = case.num_kv_heads * case.head_dim * 2
        kv_bytes = (dec_tokens + int(case.seq_lens[-1])) * 2 * row
        fl = chunk_flops(case)
        res[f"step{st}"] = {"chunk_tokens": int(case.query_lens[-1]), "call_ms": ms,
                            "call_ms_p10_p90": [flushed["p10"], flushed["p90"]], "call_ms_warm": warm["median"],
                            "decode_rows_kv_bytes": dec_tokens * 2 * row, "chunk_gflop": fl / 1e9,
                            "kv_gbs_whole_call": kv_bytes / (ms / 1e3) / 1e9,
                            "chunk_tflops_whole_call": fl / (ms / 1e3) / 1e12}
        res[f"step{st}"].update(chunk_alone(case, desc, ws, out, calls, warmup, flush))
        del case
    res["workload"] = ("long-context mixed call: 8 decodes at 32768 (+1 in step 2), decodes A (1000) and B (2000), "
                       "and a 3000-token prompt chunked 2048 + 952, 32/8 heads x 128, bf16, bs 16")
    return res


# --------------------------------------------------------------------------
# DSA dual cache: write through two views, then MLA decode per layer
# --------------------------------------------------------------------------

def run_mla(calls, warmup, flush):
    import numpy as np
    import torch
    import paged_kv_cache_130_amd as pa
    import workloads
    case = workloads.make_mla_case(device="cuda")
    bs = case.block_size
    page_mla, page_idx = bs * 656, bs * 132
    mla_v = pa.CacheView(0, page_mla, case.block_bytes, 656)
    idx_v = pa.CacheView(2 * page_mla, page_idx, case.block_bytes, 132)
    img = torch.full((case.num_blocks, case.block_bytes), 0xFF, dtype=torch.uint8, device="cuda")
    pop_slots = torch.from_numpy(case.populate_slots).cuda()
    step_slots = torch.from_numpy(case.step_slots).cuda()
    ntok = len(case.populate_slots)

    # Populate each layer's two views with packed rows (the first pass over the fresh allocation is
    # not timed), then time the populate of layer 1.
    for layer in range(2):
        pa.pa_reshape_and_cache(case.mla_rows[layer], pop_slots, img, mla_v, layer, bs, case.num_blocks,
                                v=case.idx_rows[layer], v_cache=img, v_view=idx_v)
    pop = dist(time_calls(torch, lambda: pa.pa_reshape_and_cache(
        case.mla_rows[1], pop_slots, img, mla_v, 1, bs, case.num_blocks, v=case.idx_rows[1], v_cache=img,
        v_view=idx_v), 10, flush))
    # Reference for the write rates: torch's device copy of the same bytes (the populate reads and
    # writes ntok x 788 bytes), timed the same way.
    ref_src = torch.empty(ntok * (656 + 132), dtype=torch.uint8, device="cuda").fill_(7)
    ref_dst = torch.empty_like(ref_src)
    ref = dist(time_calls(torch, lambda: ref_dst.copy_(ref_src), 10, flush))
    del ref_src, ref_dst
    # Quantize-on-write of the same populate: bf16 latent / RoPE / indexer key in, both views written.
    g = torch.Generator(device="cuda")
    g.manual_seed(1305)
    lat = torch.randn(ntok, 512, generator=g, device="cuda").to(torch.bfloat16)
    rope = torch.randn(ntok, 64, generator=g, device="cuda").to(torch.bfloat16)
    key = torch.randn(ntok, 128, generator=g, device="cuda").to(torch.bfloat16)
    qimg = torch.full_like(img, 0xFF)
    quant_call = lambda: pa.pa_quantize_and_cache_mla(lat, rope, pop_slots, qimg, mla_v, 1, bs, case.num_blocks,  # noqa: E731
                                                      index_key=key, index_cache=qimg, index_view=idx_v)
    quant_call()
    quant = dist(time_calls(torch, quant_call, 10, flush))
    del lat, rope, key, qimg
    torch.cuda.empty_cache()
    quant_bytes = ntok * ((512 + 64 + 128) * 2 + 656 + 132 + 8)
    B = len(case.context_lens)
    max_ctx = int(case.context_lens.max())
    descs = [pa.AttnDesc(kv_format=pa.PA_KV_MLA656_E4M3, num_q_heads=128, num_kv_heads=1, qk_dim=576, v_dim=512,
                         block_size=bs, num_blocks=case.num_blocks, k_view=mla_v, k_cache_bytes=img.numel(),
                         layer=layer) for layer in range(2)]
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(descs[0], B, max_ctx)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, 128, 512, dtype=torch.int16, device="cuda")
    tables = torch.from_numpy(case.block_tables).cuda()
    lens = torch.from_numpy(case.context_lens).cuda()
    for layer in range(2):   # this step's token of every sequence, both views of both layers
        pa.pa_reshape_and_cache(case.step_mla_rows[layer], step_slots, img, mla_v, layer, bs, case.num_blocks,
                                v=case.step_idx_rows[layer], v_cache=img, v_view=idx_v)
    dec = {}
    for layer in range(2):
        dec[layer] = call_stats(torch, lambda: pa.pa_decode(out, case.q, img, None, tables, lens, max_ctx, case.scale,
                                                           descs[layer], ws), flush, calls, warmup)
    dec_mean = float(np.mean([dec[l][0]["mean"] for l in range(2)]))
    dec_med = float(np.mean([dec[l][0]["median"] for l in range(2)]))
    dec_warm = float(np.mean([dec[l][1]["median"] for l in range(2)]))
    sparse = run_dsa_sparse(case, img, idx_v, descs, tables, lens, calls, warmup, flush)
    sum_ctx = int(case.context_lens.sum())
    kv = sum_ctx * 656 + B * 128 * 576 * 2 + B * 128 * 512 * 2 + int(((case.context_lens + bs - 1) // bs).sum()) * 4
    flops = sum_ctx * 128 * (576 + 512) * 2
    tf = flops / (dec_mean / 1e3) / 1e12
    traffic, traffic_src = traffic_for("dsa_mla")
    return {
        "workload": ("DSA dual cache, block-outer BLHNC, 2 layers, bs 64, 9216 blocks x 100864 B; MLA decode: 64 seqs, "
                     "ctx U[1024,8192], 128 heads on one latent head, q 512+64 bf16, fp8-e4m3 latent"),
        "sum_context_tokens": sum_ctx,
        "populate_write_ms_per_layer": pop["median"],
        "populate_write_gbs": ntok * 2 * (656 + 132) / (pop["median"] / 1e3) / 1e9,
        "populate_write_hbm_frac": ntok * 2 * (656 + 132) / (pop["median"] / 1e3) / 1e9 / HBM_PEAK_GBS,
        "device_copy_same_bytes_ms": ref["median"],
        "device_copy_same_bytes_hbm_frac": ntok * 2 * (656 + 132) / (ref["median"] / 1e3) / 1e9 / HBM_PEAK_GBS,
        "quantize_write_ms_per_layer": quant["median"],
        "quantize_write_gbs": quant_bytes / (quant["median"] / 1e3) / 1e9,
        "quantize_write_hbm_frac": quant_bytes / (quant["median"] / 1e3) / 1e9 / HBM_PEAK_GBS,
        "ms_per_step": 2 * dec_mean,
        "mla_decode_call_ms": dec_med,
        "mla_decode_call_ms_mean": dec_mean,
        "mla_decode_call_ms_p10_p90": [float(np.mean([dec[l][0]["p10"] for l in range(2)])),
                                       float(np.mean([dec[l][0]["p90"] for l in range(2)]))],
        "mla_decode_call_ms_warm": dec_warm,
        "mla_hbm_gbs": kv / (dec_mean / 1e3) / 1e9,
        "mla_hbm_frac": kv / (dec_mean / 1e3) / 1e9 / HBM_PEAK_GBS,
        "mla_counter_gbs": None if traffic is None else traffic / (dec_mean / 1e3) / 1e9,
        "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TF, "unit": "TFLOP/s",
                     "frac": tf / MFMA_BF16_PEAK_TF, "traffic": traffic, "traffic_source": traffic_src,
                     "kernel": "pa_decode (decode_mla_kernel + mla_merge_kernel)",
                     "algorithmic_flops_per_call": flops, "algorithmic_bytes_per_call": kv,
                     "duration": "mean of the flushed calls"},
        "sparse": sparse,
    }


def run_dsa_sparse(case, img, idx_v, descs, tables, lens, calls, warmup, flush):
    """DSA sparse step per layer: indexer scores + top-k (pa_indexer_topk), then MLA decode over the selection."""
    import numpy as np
    import torch
    import paged_kv_cache_130_amd as pa
    B, H, K = len(case.context_lens), case.index_heads, case.top_k
    max_ctx = int(case.context_lens.max())
    scores = torch.empty(B, max_ctx, dtype=torch.float32, device="cuda")
    pos = torch.empty(B, K, dtype=torch.int32, device="cuda")
    slots = torch.empty_like(pos)
    counts = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(descs[0], B, K)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, case.num_q_heads, 512, dtype=torch.int16, device="cuda")
    idx, dec = {}, {}
    for layer in range(2):
        idx_call = lambda: pa.pa_indexer_topk(pos, slots, counts, scores, case.q_index, case.index_weights,  # noqa: E731
                                              img, idx_v, layer, tables, lens, max_ctx, case.block_size,
                                              case.num_blocks)
        idx[layer] = call_stats(torch, idx_call, flush, calls, warmup)
        idx_call()   # this layer's selection feeds its decode
        dec[layer] = call_stats(torch, lambda: pa.pa_mla_sparse_decode(out, case.q, img, slots, counts, K, case.scale,
                                                                       descs[layer], ws), flush, calls, warmup)
    idx_ms = float(np.mean([idx[l][0]["median"] for l in range(2)]))
    dec_ms = float(np.mean([dec[l][0]["median"] for l in range(2)]))
    ctx = case.context_lens.astype(np.int64)
    sel = np.minimum(ctx, K)
    nblk = int(((ctx + case.block_size - 1) // case.block_size).sum())
    # Indexer call: index rows read once, queries and weights, table entries; scores written then re-read
    # by the selection; positions and slots written.
    idx_bytes = int(ctx.sum()) * (132 + 4 + 4) + B * H * (128 * 2 + 4) + nblk * 4 + B * K * 8
    dec_bytes = int(sel.sum()) * (656 + 4) + B * 128 * (576 + 512) * 2
    dec_flops = int(sel.sum()) * 128 * (576 + 512) * 2
    tf = dec_flops / (dec_ms / 1e3) / 1e12
    traffic, traffic_src = traffic_for("dsa_sparse")
    step_ms = 2 * (idx_ms + dec_ms)
    return {
        "workload": (f"DSA sparse decode on the same cache, per layer: lightning indexer ({H} heads x 128, bf16 "
                     f"queries, fp8 keys) over every context token, top {K} per sequence, MLA decode over the "
                     "selected slots"),
        "ms_per_step_two_layers": step_ms,
        "decode_tokens_per_s": B / (step_ms / 1e3),
        "indexer_topk_call_ms": idx_ms,
        "indexer_topk_call_ms_warm": float(np.mean([idx[l][1]["median"] for l in range(2)])),
        "indexer_topk_gbs": idx_bytes / (idx_ms / 1e3) / 1e9,
        "indexer_topk_hbm_frac": idx_bytes / (idx_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "sparse_decode_call_ms": dec_ms,
        "sparse_decode_call_ms_warm": float(np.mean([dec[l][1]["median"] for l in range(2)])),
        "sparse_decode_tflops": tf,
        "sparse_decode_mfma_frac": tf / MFMA_BF16_PEAK_TF,
        "sparse_decode_gbs": dec_bytes / (dec_ms / 1e3) / 1e9,
        "sparse_decode_traffic": traffic,
        "sparse_decode_traffic_source": traffic_src,
        "selected_tokens": int(sel.sum()),
    }


# --------------------------------------------------------------------------
# CPU baseline (the oracle on the host cores)
# --------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_sample(case, budget_s):
    """Oracle decode of whole sequences in order until `budget_s` of oracle time is spent."""
    import numpy as np
    import torch
    from oracle import attention as A
    from oracle import paging as P
    row = case.row_bytes
    ov = P.CacheView(0, 0, case.block_size * row, row)
    q = case.q.cpu().numpy().view(np.uint16)
    done_tokens, spent, seqs = 0, 0.0, 0
    for s in range(case.num_seqs):
        n = int(case.context_lens[s])
        nb = P.blocks_needed(n, case.block_size)
        ids = torch.as_tensor(case.block_tables[s, :nb].astype(np.int64), device=case.k_pool.device)
        k_img = case.k_pool.index_select(0, ids).contiguous().view(torch.uint8).reshape(-1).cpu().numpy()
        v_img = case.v_pool.index_select(0, ids).contiguous().view(torch.uint8).reshape(-1).cpu().numpy()
        t0 = time.perf_counter()
        A.paged_decode(q[s:s + 1], case.dtype, k_img, ov, v_img, ov, 0, np.arange(nb)[None, :], [n], case.block_size,
                       case.num_kv_heads, case.head_dim, case.scale)
        spent += time.perf_counter() - t0
        done_tokens += n
        seqs += 1
        if spent >= budget_s:
            break
    return {"value": round(done_tokens * 2 * row / spent / 1e9, 4), "unit": "GB/s",
            "sample": f"{seqs} of {case.num_seqs} sequences (all {case.num_q_heads} heads), {done_tokens} tokens, "
                      f"{spent:.1f} s of oracle time; decode tokens/s {seqs / spent:.2f}"}


def cpu_baseline(case, budget_s: float = 12.0, single_budget_s: float = 8.0):
    """The oracle (NumPy fp64) on the host cores over a bounded sample of the batch: with the BLAS
    threads fixed at start-up, then with one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    r = oracle_sample(case, budget_s)
    with threadpool_limits(limits=1):
        one = oracle_sample(case, single_budget_s)
    return {**r, "cores": int(threads), "kind": "oracle", "cpu_model": cpu_model(),
            "host_cpus_visible": len(os.sched_getaffinity(0)),
            "threads_note": "cores = BLAS threads of the oracle's NumPy (OMP/OPENBLAS_NUM_THREADS set before import)",
            "single_core": {**one, "cores": 1}}


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_dispatch": n, "bytes_written_per_dispatch": n}))


def rounded(x):
    if isinstance(x, float):
        return round(x, 4)
    if isinstance(x, dict):
        return {k: rounded(v) for k, v in x.items()}
    if isinstance(x, list):
        return [rounded(v) for v in x]
    return x


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (one MI355X). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_kv_cache_130_amd  # noqa: F401  (fails loudly if libpa.so is missing)

    if args.calibrate_copy:
        calibrate_copy()
        return
    torch.cuda.set_device(0)
    flush = Flush(torch, args.flush)

    metric = "paged decode effective KV GB/s (% of HBM peak) and decode tokens/s at 1 GPU"
    res = {"metric": metric, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded N(0,1) K/V/Q, seeded block tables)",
           "timing": f"cache flush ({FLUSH_BYTES >> 20} MiB {args.flush}) before every timed call, outside its "
                     f"events; call figures are medians of >= {MIN_CALLS} calls"}
    if args.workload in ("mha13b", "gqa_prefix", "gqa_prefix_copied", "long_decode", "mha13b_fp8",
                         "gqa_prefix_copied_fp8"):
        case, r = run_dense(args.workload, args.steps, args.warmup, args.partition, flush)
        res.update({"value": r["value"], "unit": "GB/s", "ms_per_step": r["ms_per_step"], "dtype": r["dtype"],
                    "config": dict(workload=r["workload"], **r["config"])})
        res.update({k: v for k, v in r.items() if k not in ("value", "ms_per_step", "dtype", "config", "workload")})
        if not args.no_cpu_baseline and case.k_pool is not None:
            res["cpu_baseline"] = cpu_baseline(case)
        del case
        torch.cuda.empty_cache()
    elif args.workload == "long_mixed":
        r = run_mixed(max(MIN_CALLS, args.steps), args.warmup, flush)
        res.update({"value": r["step1"]["kv_gbs_whole_call"], "unit": "GB/s", "ms_per_step": r["step1"]["call_ms"],
                    "dtype": "bf16", "config": {"workload": r["workload"]}, "steps_detail": r})
    elif args.workload.startswith("prefill_chunk"):
        r = run_chunk_only(1 if args.workload.endswith("2048") else 2, max(MIN_CALLS, args.steps), args.warmup, flush)
        res.update({"value": r["chunk_alone_tflops"], "unit": "TFLOP/s", "ms_per_step": r["chunk_alone_ms"],
                    "dtype": "bf16", "config": {"workload": r["workload"]},
                    "roofline": {"bound": "mfma", "achieved": r["chunk_alone_tflops"], "peak": MFMA_BF16_PEAK_TF,
                                 "unit": "TFLOP/s", "frac": r["chunk_alone_mfma_frac"], "traffic": None,
                                 "kernel": "mixed_chunk_kernel (chunk rows only)",
                                 "algorithmic_flops_per_call": r["chunk_gflop"] * 1e9},
                    "chunk_detail": r})
    else:
        r = run_mla(max(MIN_CALLS, args.steps), args.warmup, flush)
        res.update({"value": r["mla_hbm_gbs"], "unit": "GB/s", "ms_per_step": r["ms_per_step"], "dtype": "bf16",
                    "config": {"workload": r["workload"]}, "roofline": r["roofline"], "mla_detail": r})

    if args.workload == "mha13b" and not args.no_extra:
        extra = {}
        for name in ("gqa_prefix_copied", "gqa_prefix", "long_decode", "mha13b_fp8", "gqa_prefix_copied_fp8"):
            case, r = run_dense(name, 10, 3, 0, flush)
            extra[name] = {"workload": r["workload"], "decode_call_ms": r["decode_call_ms"],
                           "decode_call_ms_mean": r["decode_call_ms_mean"],
                           "decode_call_ms_p10_p90": r["decode_call_ms_p10_p90"],
                           "decode_call_ms_warm": r["decode_call_ms_warm"],
                           "kv_gbs": r["roofline"]["achieved"], "frac_of_hbm_peak": r["roofline"]["frac"],
                           "kv_gbs_logical": r["decode_kv_gbs_logical"], "kv_gbs_counter": r["decode_kv_gbs_counter"],
                           "traffic_source": r["roofline"]["traffic_source"],
                           "decode_tokens_per_s": r["decode_tokens_per_s"]}
            for k in ("copy_on_write_pairs", "copy_on_write_ms", "copy_on_write_gbs", "quantize_pool_ms",
                      "quantize_pool_gbs"):
                if k in r:
                    extra[name][k] = r[k]
            del case
            torch.cuda.empty_cache()
        extra["long_mixed"] = run_mixed(MIN_CALLS, 3, flush)
        torch.cuda.empty_cache()
        m = run_mla(MIN_CALLS, 3, flush)
        extra["dsa_mla"] = {k: m[k] for k in ("workload", "sum_context_tokens", "populate_write_ms_per_layer",
                                              "populate_write_gbs", "populate_write_hbm_frac",
                                              "device_copy_same_bytes_hbm_frac", "quantize_write_ms_per_layer",
                                              "quantize_write_gbs", "quantize_write_hbm_frac", "mla_decode_call_ms",
                                              "mla_decode_call_ms_mean", "mla_decode_call_ms_p10_p90",
                                              "mla_decode_call_ms_warm", "mla_hbm_gbs", "mla_hbm_frac",
                                              "mla_counter_gbs")}
        extra["dsa_mla"]["mfma_tflops"] = m["roofline"]["achieved"]
        extra["dsa_mla"]["mfma_frac"] = m["roofline"]["frac"]
        extra["dsa_sparse"] = m["sparse"]
        res["extra"] = extra
    print(json.dumps(rounded(res)), flush=True)


if __name__ == "__main__":
    main()

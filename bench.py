"""Benchmark of the paged-KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mha13b|gqa_prefix|gqa_prefix_copied|long_decode]

One step = one pass of the decode hot path over one batch: pa_reshape_and_cache writes each
sequence's new K/V row through slot_mapping, then pa_decode attends every sequence to its whole
paged context. Inputs are seeded synthetic draws already resident in HBM when timing starts.

The JSON line reports the whole step's algorithmic bytes per second as `value`, with decode tokens/s
beside it. `roofline` covers the pa_decode call (the dominant kernel): its algorithmic bytes divided
by its own duration, from HIP events recorded on the launch stream around every call in the timed
region. `cpu_baseline` times the NumPy oracle on the host cores over a bounded sample of the same
batch.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode_dense.hip", "decode_mfma.hip", "decode_common.h", "pa_device.h", "pa_internal.h", "api.hip"):
        with open(os.path.join(ROOT, "paged_kv_cache_130_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mha13b",
                    choices=["mha13b", "gqa_prefix", "gqa_prefix_copied", "long_decode"])
    ap.add_argument("--partition", type=int, default=0, help="pa_decode partition_size (0: library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


def build_workload(name: str):
    import workloads
    if name == "mha13b":
        case = workloads.make_dense_case("mha13b", device="cuda")
        desc_name = "13B-shaped MHA decode: 64 seqs, ctx U[128,2048], 40/40 heads x 128, fp16, bs 16, 12288 blocks"
    elif name in ("gqa_prefix", "gqa_prefix_copied"):
        case = workloads.make_dense_case("gqa_prefix", device="cuda", copied_prefix=name.endswith("copied"))
        desc_name = ("GQA decode, 256 seqs sharing a 2000-token prompt (125 blocks) + lognormal suffix, 32/8 heads x "
                     "128, bf16, bs 16" + (", prompt blocks copied per sequence" if name.endswith("copied") else ""))
    else:
        case = workloads.make_dense_case("tiny", seed=1304, context_lens=[32768] * 8, num_blocks=17408,
                                         num_q_heads=32, num_kv_heads=8, dtype="bf16", device="cuda")
        desc_name = "long-context decode: 8 seqs x 32768 tokens, 32/8 heads x 128, bf16, bs 16, partitions of 512"
    return case, desc_name


def algorithmic_bytes(case):
    """Bytes the method must move (distinct rows read once), for the decode call and for the cache write."""
    import numpy as np
    ctx = case.context_lens.astype(np.int64)
    row = case.row_bytes
    head_bytes = case.head_dim * 2
    B, Hq = case.num_seqs, case.num_q_heads
    # distinct (block, position) rows touched: shared prompt blocks count once
    if case.extra.get("shared_prefix_blocks") and not case.extra.get("copied_prefix"):
        shared_tokens = case.extra["shared_prefix_blocks"] * case.block_size
        unique_tokens = int(ctx.sum() - (B - 1) * shared_tokens)
    else:
        unique_tokens = int(ctx.sum())
    nblk = int(((ctx + case.block_size - 1) // case.block_size).sum())   # block-table entries read
    fixed = B * Hq * head_bytes * 2 + nblk * 4 + B * 4            # q + out + block-table entries + lengths
    decode_logical = int(ctx.sum()) * 2 * row + fixed
    decode_unique = unique_tokens * 2 * row + fixed
    write = B * (2 * row) * 2 + B * 8                              # read + write of K and V rows, slots
    return decode_logical, decode_unique, write


def cpu_baseline(case, budget_s: float = 15.0):
    """Oracle (NumPy fp64) on the host over a bounded sample: whole sequences in order until the budget."""
    import numpy as np
    import torch
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
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
        tbl = np.arange(nb)[None, :]
        t0 = time.perf_counter()
        A.paged_decode(q[s:s + 1], case.dtype, k_img, ov, v_img, ov, 0, tbl, [n], case.block_size,
                       case.num_kv_heads, case.head_dim, case.scale)
        spent += time.perf_counter() - t0
        done_tokens += n
        seqs += 1
        if spent >= budget_s:
            break
    gbs = done_tokens * 2 * row / spent / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{seqs} of {case.num_seqs} sequences (all {case.num_q_heads} heads), {done_tokens} tokens, "
                      f"{spent:.1f} s of oracle time; decode tokens/s {seqs / spent:.2f}"}


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_dispatch": n, "bytes_written_per_dispatch": n}))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build runs on a single MI355X (no multi-GPU path). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import paged_kv_cache_130_amd as pa

    if args.calibrate_copy:
        calibrate_copy()
        return

    torch.cuda.set_device(0)
    case, wdesc = build_workload(args.workload)
    B, Hq, D = case.num_seqs, case.num_q_heads, case.head_dim
    kd, vd = case.k_pool, case.v_pool
    view = pa.dense_view(case.block_size, case.num_kv_heads, D)
    partition = args.partition or (512 if args.workload == "long_decode" else 0)
    desc = pa.dense_desc(case.dtype, Hq, case.num_kv_heads, D, case.block_size, case.num_blocks, kd.numel() * 2,
                         vd.numel() * 2, partition)
    max_ctx = int(case.context_lens.max())
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, B, max_ctx)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, D, dtype=torch.int16, device="cuda")
    q = case.q
    tables = torch.from_numpy(case.block_tables).cuda()
    lens = torch.from_numpy(case.context_lens).cuda()
    slots = torch.from_numpy(case.new_slots).cuda()
    new_k, new_v = case.new_k, case.new_v
    stream = torch.cuda.current_stream()

    def step(ev=None):
        pa.pa_reshape_and_cache(new_k, slots, kd, view, 0, case.block_size, case.num_blocks, v=new_v, v_cache=vd,
                                v_view=view)
        if ev is not None:
            ev[0].record(stream)
        pa.pa_decode(out, q, kd, vd, tables, lens, max_ctx, case.scale, desc, ws)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    dec_ms = [a.elapsed_time(b) for a, b in events]
    dec_ms_mean = float(np.mean(dec_ms))

    logical, unique, write = algorithmic_bytes(case)
    value = (unique + write) / (ms_step / 1e3) / 1e9
    achieved = unique / (dec_ms_mean / 1e3) / 1e9
    traffic = None
    if os.path.exists(COUNTERS):
        with open(COUNTERS) as f:
            cnt = json.load(f)
        e = cnt.get(args.workload)
        if e and e.get("kernel_hash") == kernel_source_hash():
            traffic = e.get("hbm_bytes_per_call")
    res = {
        "metric": "paged decode effective KV GB/s (% of HBM peak) and decode tokens/s at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded block tables)",
        "config": {"workload": wdesc, "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": case.num_kv_heads,
                   "head_dim": D, "block_size": case.block_size, "num_blocks": case.num_blocks,
                   "sum_context_tokens": int(case.context_lens.sum()), "partition_size": partition or "auto"},
        "decode_tokens_per_s": round(B / (ms_step / 1e3), 1),
        "decode_call_ms": round(dec_ms_mean, 4),
        "decode_call_ms_p10_p90": [round(float(np.percentile(dec_ms, 10)), 4),
                                   round(float(np.percentile(dec_ms, 90)), 4)],
        "decode_kv_gbs_logical": round(logical / (dec_ms_mean / 1e3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "pa_decode (decode_dense_kernel + decode_reduce_kernel)",
                     "algorithmic_bytes_per_call": unique},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

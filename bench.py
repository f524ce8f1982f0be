"""Benchmark of the INT4 paged KV-cache hot path on one MI355X.

Workload: long-context decode, 4 sequences x 131072 tokens, 64 query heads,
8 KV heads, head_size 128, bf16 inputs, split-K over 64 segments.  One step =
write the new token of every sequence into the packed cache (int4_kv_write),
then one decode step of causal paged attention over the full context
(int4_paged_attention: split-K kernel + segment reduction).  Several
independent caches are rotated between steps so that no step reads a cache
still resident in the 256 MB Infinity Cache.

Prints one JSON line: decode effective KV GB/s (packed K+V bytes of every key
attended, once per KV head, over the step time), the bulk cache-write rate
(tokens/s, from a timed full-cache fill), the roofline of the decode kernels
(HIP events on the launch stream), and the CPU oracle timed on a bounded
sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import int4_quantized_paged_amd as ik  # noqa: E402
from int4_quantized_paged_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "decode attn effective KV GB/s (% of HBM peak); int4 cache-write tokens/s"
NUM_SEGMENTS = 64


def _traffic_from_profiles(kernel_hash: str):
    """Measured HBM bytes per launch, if the committed counter summary was taken
    on the current kernel source."""
    p = os.path.join(HERE, "profiles", "decode_long_context_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256") != kernel_hash:
        return None
    return d.get("hbm_bytes_per_attention_call")


def _kernel_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("decode_lds.hip", "decode.hip", "device_common.h", "launch.h"):
        with open(os.path.join(HERE, "int4_quantized_paged_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def build_buffers(nbufs: int, dev: str):
    bufs = []
    for i in range(nbufs):
        w = wl.long_context_decode(device=dev, seed=3 + 1000 * i)
        cache = ik.empty_cache(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)
        idx_new, slots_new = w.token_set("new")
        idx_all, slots_all = w.token_set("all")
        signs = w.signs.to(dev)
        slots_all_d = slots_all.to(dev)
        # set-up: fill the whole cache (prior context and the new tokens)
        ik.int4_kv_write(w.key, w.value, slots_all_d, cache, signs)
        b = dict(w=w, cache=cache, signs=signs, key_new=w.key[idx_new.to(dev)].contiguous(),
                 value_new=w.value[idx_new.to(dev)].contiguous(), slots_new=slots_new.to(dev),
                 query=w.query, cu=w.cu_seqlens_q().to(dev), su=w.seqused_k().to(dev),
                 bt=w.block_table.to(dev),
                 segs=ik.segment_buffers(w.num_seqs, w.num_q_heads, NUM_SEGMENTS, w.head_size, dev),
                 out=torch.empty_like(w.query))
        if i == 0:
            b["bulk"] = (w.key, w.value, slots_all_d)  # kept for the write-rate measurement
        else:
            del w.key, w.value
        bufs.append(b)
    torch.cuda.synchronize()
    return bufs


def step(b, ev=None):
    ik.int4_kv_write(b["key_new"], b["value_new"], b["slots_new"], b["cache"], b["signs"])
    w = b["w"]
    if ev is not None:
        ev[0].record()
    ik.int4_paged_attention(b["query"], b["cache"], b["cu"], b["su"], 1, w.max_seqlen_k, b["bt"],
                            w.softmax_scale, b["signs"], out=b["out"], num_segments=NUM_SEGMENTS,
                            segm_output=b["segs"][0], segm_max=b["segs"][1],
                            segm_expsum=b["segs"][2])
    if ev is not None:
        ev[1].record()


def measure_bulk_write(b, reps: int = 5):
    key, value, slots = b["bulk"]
    cache = torch.empty_like(b["cache"])
    ik.int4_kv_write(key, value, slots, cache, b["signs"])
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ik.int4_kv_write(key, value, slots, cache, b["signs"])
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
    times.sort()
    t = times[len(times) // 2]
    T = key.shape[0]
    return T / t, t, T


def cpu_baseline(b):
    """The oracle (plain single-threaded C) on a bounded sample of the same
    workload: one of the 4 sequences, its 131072 tokens encoded, then one
    decode query of all 64 heads attended over them."""
    import numpy as np
    import oracle
    oracle._load()
    w = b["w"]
    key, value, _ = b["bulk"]
    L = w.kv_lens[0]
    sub = wl.Workload(w.name + " seq 0", w.dtype, w.num_q_heads, w.num_kv_heads, w.head_size,
                      w.num_blocks, [L], [1], [1], w.block_table[:1].clone(), key[:L], value[:L],
                      w.query[:1], w.signs)
    kb, vb = wl.bits16(sub.key), wl.bits16(sub.value)
    qb = wl.bits16(sub.query)
    _, slots = sub.token_set("all")
    cache = np.zeros(oracle.cache_shape(w.num_blocks, 16, w.num_kv_heads, w.head_size), np.uint8)
    t0 = time.perf_counter()
    oracle.kv_write(kb, vb, "bf16", slots.numpy(), cache, w.signs.numpy())
    t_write = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.attention_plain(qb, "bf16", cache, sub.cu_seqlens_q().numpy(), sub.seqused_k().numpy(),
                           sub.block_table.numpy(), w.softmax_scale, w.signs.numpy(), w.num_q_heads)
    t_attn = time.perf_counter() - t0
    kv = sub.kv_bytes_attended()
    return {"value": kv / t_attn / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"1 of 4 sequences (131072 keys x 8 KV heads, 64 query heads): plain fp64 "
                      f"attention {t_attn:.2f} s; its cache write {t_write:.2f} s",
            "write_tokens_per_s": L / t_write}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the INT4 KV-cache path is built and measured on a "
              "single MI355X (multi-GPU sharding is a design note only); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"
    if args.calibrate_copy:
        n = 1 << 28  # 2^28 fp32 = 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 4 * n, "copies": 4}), flush=True)
        return
    ik.load_library()
    nbufs = 2  # 2 x 570 MB > 256 MB Infinity Cache
    bufs = build_buffers(nbufs, dev)
    w = bufs[0]["w"]
    kv_bytes = w.kv_bytes_attended()

    for i in range(args.warmup):
        step(bufs[i % nbufs])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(bufs[i % nbufs], evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    attn_s = sum(a.elapsed_time(b) for a, b in evs) / 1e3 / args.steps

    wr_tps, wr_t, wr_T = measure_bulk_write(bufs[0])
    value = kv_bytes / (ms_per_step / 1e3) / 1e9
    achieved = kv_bytes / attn_s / 1e9
    traffic = _traffic_from_profiles(_kernel_hash())
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16 mfma/f32",
        "data": "synthetic",
        "config": {"workload": "long-context decode: 4 seqs x 131072 tokens, 64 q / 8 KV heads, "
                               "head_size 128, bf16 K/V/Q N(0,1), block_size 16, split-K 64 "
                               "segments + segment reduction; step = write 4 new tokens + decode",
                   "global_batch": 4, "seq_len": 131072, "parallelism": "none (1 GPU)"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "write_tokens_per_s": round(wr_tps, 1),
        "write_bulk": {"tokens": wr_T, "seconds": wr_t,
                       "GB_per_s": round(w.write_bytes("all") / wr_t / 1e9, 1)},
        "roofline": {"kernel": "decode_lds_kernel + reduce_kernel (one int4_paged_attention call)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": kv_bytes,
                     "avg_launch_us": round(attn_s * 1e6, 2)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(bufs[0])
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

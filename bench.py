"""Benchmark of the INT4 paged KV-cache hot path on one MI355X.

Workload: long-context decode, 4 sequences x 131072 tokens, 64 query heads,
8 KV heads, head_size 128, bf16 inputs, split-K over 64 segments.  One step =
write the new token of every sequence into the packed cache, then one decode
step of causal paged attention over the full context: int4_decode_step, which
does both in the split-K launch (the workgroup that reads a new token's block
encodes and stores it first) followed by the segment reduction;
`--separate-calls` times int4_kv_write + int4_paged_attention instead (same
bytes and output, one more launch).  Two independent
caches alternate between steps so that no step reads a cache still resident
in the 256 MB Infinity Cache.

Steps are plain library calls: the host enqueues a step in about a fifth of
its GPU time, and HIP-graph replays of the same calls (`--graph`, checked bit
for bit against plain calls) measured a few microseconds slower per step.
Before the warm-up steps, about 1 s of untimed steps bring the GPU to its
steady clock and address-translation state (the first few hundred steps on
a fresh process run up to 15% slower, and the launch time eases by another
2-3% over the next half second); the JSON line reports how many.  The
timed steps run back to back (an event recorded between two calls is a
queue packet of its own and costs each call 2-3 us); a second pass of the
same steps, and of the attention calls, with an event after each call gives
the per-call first five, median, mean and last five.
Prints one JSON line: decode
effective KV GB/s (packed K+V bytes of every key attended, once per KV head,
over the step time), the bulk cache-write rate (tokens/s, from a timed
full-cache fill), the roofline of the attention call (HIP events on the
launch stream around back-to-back calls), and the CPU oracle timed on the
same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import int4_quantized_paged_amd as ik  # noqa: E402
from int4_quantized_paged_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
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
    for f in ("decode_lds.hip", "decode.hip", "device_common.h", "launch.h", "encode_row.h"):
        with open(os.path.join(HERE, "int4_quantized_paged_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


def write_new(b):
    ik.int4_kv_write(b["key_new"], b["value_new"], b["slots_new"], b["cache"], b["signs"])


def attend(b):
    w = b["w"]
    ik.int4_paged_attention(b["query"], b["cache"], b["cu"], b["su"], 1, w.max_seqlen_k, b["bt"],
                            w.softmax_scale, b["signs"], out=b["out"], num_segments=NUM_SEGMENTS,
                            segm_output=b["segs"][0], segm_max=b["segs"][1],
                            segm_expsum=b["segs"][2])


def step(b):
    """One decode step in one launch: the new tokens' rows are encoded by the
    workgroups that read their blocks (int4_decode_step)."""
    w = b["w"]
    ik.int4_decode_step(b["key_new"], b["value_new"], b["slots_new"], b["query"], b["cache"],
                        b["cu"], b["su"], 1, w.max_seqlen_k, b["bt"], w.softmax_scale,
                        b["signs"], out=b["out"], num_segments=NUM_SEGMENTS,
                        segm_output=b["segs"][0], segm_max=b["segs"][1],
                        segm_expsum=b["segs"][2])


def step_separate(b):
    write_new(b)
    attend(b)


def capture(fn):
    """Record fn's library calls into a HIP graph (torch.cuda.graph makes the
    capturing stream current, which is the stream the binding passes)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def check_replay(bufs, graphs):
    """Replays must reproduce the eager result bit for bit (deterministic kernels)."""
    for b, g in zip(bufs, graphs):
        b["out"].zero_()
        attend(b)
        torch.cuda.synchronize()
        ref = b["out"].clone()
        for _ in range(2):
            b["out"].zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(b["out"], ref):
                raise RuntimeError("graph replay differs from the eager attention call")


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


def measure_stream_ceiling(read_bytes: int, write_bytes: int, reps: int = 5):
    """A plain streaming kernel with the bulk write's read:write byte mix (no
    arithmetic beyond XOR), timed like the write: the bandwidth an HBM pass of
    that mix attains, which the write is compared against."""
    read_bytes -= read_bytes % 16
    write_bytes -= write_bytes % 16
    src = torch.empty(read_bytes, dtype=torch.uint8, device="cuda").random_(0, 256)
    dst = torch.empty(write_bytes, dtype=torch.uint8, device="cuda")
    ik.int4kv_stream_rw(src, read_bytes, dst, write_bytes)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ik.int4kv_stream_rw(src, read_bytes, dst, write_bytes)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
    times.sort()
    t = times[len(times) // 2]
    del src, dst
    return t, read_bytes, write_bytes


def gather_only(bufs, n: int):
    """The attention call's block gather on its own (int4kv_stream_blocks): the
    same blocks in the same order over the same workgroups (one per sequence
    and segment) and the same LDS ring, nothing computed; n back-to-back calls
    alternating the caches, HIP events around them.  Microseconds per call:
    the rate the decode kernel's access pattern attains by itself."""
    runs = []
    for b in bufs:
        w = b["w"]
        nblk = {(L + 15) // 16 for L in w.kv_lens}
        assert len(nblk) == 1, "one block count for every sequence"
        nblk = nblk.pop()
        assert nblk % NUM_SEGMENTS == 0 and (nblk // NUM_SEGMENTS) % 2 == 0
        ids = b["bt"][:, :nblk].contiguous().view(-1)
        block_bytes = 2 * 16 * w.num_kv_heads * (w.head_size // 2 + 4)
        runs.append(lambda b=b, ids=ids, bb=block_bytes, nwg=w.num_seqs * NUM_SEGMENTS:
                    ik.int4kv_stream_blocks(b["cache"], bb, ids, nwg))
    for i in range(2 * len(runs)):
        runs[i % len(runs)]()
    _, ms = timed_block(runs, len(runs), n)
    return ms * 1e3 / n


def _median_event_us(fn, reps, rounds=5):
    """Per-call time of `reps` back-to-back calls between two HIP events on the
    launch stream (as the headline attention figure), median of `rounds`."""
    ts = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / reps)
    ts.sort()
    return ts[len(ts) // 2]


def settle(run, nbufs: int, seconds: float = 1.0, max_steps: int = 20000) -> dict:
    """Untimed steps until the GPU reaches its steady clock and address-
    translation state (about 1 s of the same work): on a fresh process the
    first few hundred decode launches run up to 15% slower, and the launch
    time keeps easing by 2-3% over the next half second.  Done before the
    warm-up steps."""
    t0 = time.perf_counter()
    n = 0
    while n < max_steps:
        for _ in range(50):
            run[n % nbufs]()
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    return {"steps": n, "seconds": round(time.perf_counter() - t0, 3)}


def timed_calls(run, nbufs: int, n: int):
    """n calls, each followed by a HIP event recorded on the current stream (the
    stream the library launches on).  Returns (wall seconds around the n calls,
    bracketed by synchronisation, per-call event milliseconds of calls 2..n).
    The first call's interval would start on an idle GPU and include the
    host's launch latency after the synchronisation that opens the timed
    region (it is in the wall time), so the per-call times start at the
    second call: each is the time from the end of one call to the end of the
    next, i.e. a call's GPU time plus its dispatch gap."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        run[i % nbufs]()
        ev[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [ev[i].elapsed_time(ev[i + 1]) for i in range(n - 1)]


def timed_block(run, nbufs: int, n: int):
    """n calls with nothing between them, bracketed by synchronisation: the
    wall seconds, and the milliseconds between two HIP events recorded on the
    launch stream right before the first call and right after the last one.
    (An event recorded between calls is a packet of its own in the queue and
    costs the calls 2-3 us each, so the per-call statistics come from a
    separate pass of the same calls.)"""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(n):
        run[i % nbufs]()
    e1.record()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, e0.elapsed_time(e1)


def call_stats(ms):
    """First 5, median, mean and last 5 of per-call times (microseconds; calls
    2..n of a timed region)."""
    us = [x * 1e3 for x in ms]
    srt = sorted(us)
    return {"first5_us": [round(x, 2) for x in us[:5]], "median_us": round(srt[len(srt) // 2], 2),
            "mean_us": round(sum(us) / len(us), 2), "last5_us": [round(x, 2) for x in us[-5:]],
            "min_us": round(srt[0], 2), "max_us": round(srt[-1], 2)}


def _graph_us(fn, n):
    """Per-call time of `n` calls of fn captured in one HIP graph and replayed
    (median of five rounds of 5 replays): the GPU's time for the calls without
    the host's per-call cost.  The library's kernels record no memsets."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    return _median_event_us(g.replay, 5) / n


def _attention_setup(w, dev, ns, ncaches=1):
    caches = [ik.empty_cache(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)]
    _, slots = w.token_set("all")
    signs = w.signs.to(dev)
    ik.int4_kv_write(w.key, w.value, slots.to(dev), caches[0], signs)
    for _ in range(ncaches - 1):
        caches.append(caches[0].clone())
    cu, su, bt = w.cu_seqlens_q().to(dev), w.seqused_k().to(dev), w.block_table.to(dev)
    segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size, dev) if ns > 1 else \
        (None, None, None)
    out = torch.empty_like(w.query)
    state = {"i": 0}

    def call():
        c = caches[state["i"] % len(caches)]
        state["i"] += 1
        ik.int4_paged_attention(w.query, c, cu, su, w.max_seqlen_q, w.max_seqlen_k, bt,
                                w.softmax_scale, signs, out=out, num_segments=ns,
                                segm_output=segs[0], segm_max=segs[1], segm_expsum=segs[2])
    call.caches, call.signs = caches, signs
    return call


def other_rows(dev):
    """The other timed rows of the path, each at its full size: prefill on the
    chunked-prefill mix (MFMA-bound; TFLOP/s against the dense f16 peak), the
    GQA decode step (8 short sequences, latency-bound) and decode on the
    Llama-3-8B-shaped batch (HBM-bound; two cache copies alternate).
    Back-to-back calls between HIP events, median of five rounds."""
    rows = {}
    for d in (128, 64):
        w = wl.chunked_prefill(device=dev, head_size=d)
        call = _attention_setup(w, dev, 1)
        for _ in range(3):
            call()
        us = _median_event_us(call, 10)
        fl = w.attention_flops()
        # the mix's step as a whole: write its new tokens (sum of q_b), then attend
        idx_n, slots_n = w.token_set("new")
        kn, vn = w.key[idx_n.to(dev)].contiguous(), w.value[idx_n.to(dev)].contiguous()
        sn = slots_n.to(dev)
        cache0, sg = call.caches[0], call.signs

        def write_new():
            ik.int4_kv_write(kn, vn, sn, cache0, sg)

        def write_and_attend():
            write_new()
            call()
        for _ in range(3):
            write_and_attend()
        us_w = _median_event_us(write_new, 10)
        us_wa = _median_event_us(write_and_attend, 10)
        rows[f"prefill_d{d}"] = {
            "workload": f"chunked-prefill mix: 32 seqs, {sum(w.query_lens)} query tokens, "
                        f"{sum(w.kv_lens)} keys, 32 q / 8 KV heads, d {d}",
            "us": round(us, 2), "tflops": round(fl / us / 1e6, 1),
            "mfma_frac": round(fl / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4),
            "algorithmic_gflop": round(fl / 1e9, 2),
            "kv_GBps": round(w.kv_bytes_attended() / us / 1e3, 1),
            "write_new_tokens": int(idx_n.numel()), "write_us": round(us_w, 2),
            "write_GBps": round(w.write_bytes("new") / us_w / 1e3, 1),
            "write_plus_attention_us": round(us_wa, 2)}
        del w, call, kn, vn
    # the same mix over the INT8 per-token-head cache (d 128)
    w = wl.chunked_prefill(device=dev, head_size=128)
    c8 = torch.empty(ik.cache_shape_int8(w.num_blocks, w.num_kv_heads, 128), dtype=torch.uint8,
                     device=dev)
    _, slots = w.token_set("all")
    ik.int8_kv_write(w.key, w.value, slots.to(dev), c8)
    q, cu, su, bt = w.query, w.cu_seqlens_q().to(dev), w.seqused_k().to(dev), w.block_table.to(dev)
    out = torch.empty_like(q)

    def call8():
        ik.int8_paged_attention(q, c8, cu, su, w.max_seqlen_q, w.max_seqlen_k, bt,
                                w.softmax_scale, out=out)
    for _ in range(3):
        call8()
    us = _median_event_us(call8, 10)
    fl = w.attention_flops()
    rows["prefill_int8_d128"] = {
        "workload": f"chunked-prefill mix over the INT8 cache: {sum(w.query_lens)} query tokens, "
                    f"{sum(w.kv_lens)} keys, 32 q / 8 KV heads, d 128",
        "us": round(us, 2), "tflops": round(fl / us / 1e6, 1),
        "mfma_frac": round(fl / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)}
    del c8
    # ... and over the INT2 Lloyd-Max cache
    sg2 = w.signs.to(dev)
    c2 = ik.empty_cache_int2(w.num_blocks, w.num_kv_heads, 128, device=dev)
    ik.int2_kv_write(w.key, w.value, slots.to(dev), c2, sg2)

    def call2():
        ik.int2_paged_attention(q, c2, cu, su, w.max_seqlen_q, w.max_seqlen_k, bt,
                                w.softmax_scale, sg2, out=out)
    for _ in range(3):
        call2()
    us = _median_event_us(call2, 10)
    rows["prefill_int2_d128"] = {
        "workload": f"chunked-prefill mix over the INT2 cache: {sum(w.query_lens)} query tokens, "
                    f"{sum(w.kv_lens)} keys, 32 q / 8 KV heads, d 128",
        "us": round(us, 2), "tflops": round(fl / us / 1e6, 1),
        "mfma_frac": round(fl / us / 1e6 / MFMA_F16_PEAK_TFLOPS, 4)}
    del w, c2, q, out
    # GQA decode: 8 sequences of 1..1024 keys, one new token each, in one
    # int4_decode_step (latency-bound: reported in us and GB/s, not against HBM peak)
    w = wl.gqa_decode(device=dev)
    cache = ik.empty_cache(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)
    signs = w.signs.to(dev)
    idx_p, slots_p = w.token_set("prior")
    ik.int4_kv_write(w.key[idx_p.to(dev)], w.value[idx_p.to(dev)], slots_p.to(dev), cache, signs)
    idx_n, slots_n = w.token_set("new")
    kn, vn, sn = w.key[idx_n.to(dev)].contiguous(), w.value[idx_n.to(dev)].contiguous(), slots_n.to(dev)
    ns = ik.int4kv_decode_num_segments(w.num_seqs, w.num_kv_heads, w.max_seqlen_k)
    segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size, dev) if ns > 1 else \
        (None, None, None)
    cu, su, bt = w.cu_seqlens_q().to(dev), w.seqused_k().to(dev), w.block_table.to(dev)
    out = torch.empty_like(w.query)
    gstep = lambda: ik.int4_decode_step(kn, vn, sn, w.query, cache, cu, su, 1, w.max_seqlen_k,  # noqa: E731
                                        bt, w.softmax_scale, signs, out=out, num_segments=ns,
                                        segm_output=segs[0], segm_max=segs[1],
                                        segm_expsum=segs[2])
    for _ in range(20):
        gstep()
    us_plain = _median_event_us(gstep, 50)
    us = _graph_us(gstep, 20)
    rows["gqa_decode_step"] = {
        "workload": f"8 seqs, {sum(w.kv_lens)} keys in all (1..1024 each), 32 q / 8 KV heads, "
                    "d 128; write 8 new tokens + decode (int4_decode_step)",
        "num_segments": ns, "us": round(us, 2), "us_plain_calls": round(us_plain, 2),
        "timing": "us: 20 steps replayed from one HIP graph, per step (GPU time; plain calls "
                  "from Python are bound by the host's call rate at this size)",
        "kv_GBps": round(w.kv_bytes_attended() / us / 1e3, 1)}
    del w, cache, gstep

    # serving stand-in: 100 prompts of 512 tokens written (timed), then one
    # decode step per sequence at a context in [512, 640] (int4_decode_step)
    w = wl.serving_standin(device=dev)
    cache = ik.empty_cache(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)
    signs = w.signs.to(dev)
    off = w.token_offsets()
    P = 512
    pos = torch.arange(P, dtype=torch.int64)
    pidx = torch.cat([pos + off[b] for b in range(w.num_seqs)]).to(dev)
    pslots = torch.cat([w.slots_of(b, pos) for b in range(w.num_seqs)]).to(dev)
    kp, vp = w.key[pidx].contiguous(), w.value[pidx].contiguous()
    pwrite = lambda: ik.int4_kv_write(kp, vp, pslots, cache, signs)  # noqa: E731
    for _ in range(3):
        pwrite()
    pw_us = _median_event_us(pwrite, 10)
    mid = [(torch.arange(P, L - 1, dtype=torch.int64), b) for b, L in enumerate(w.kv_lens) if L - 1 > P]
    midx = torch.cat([m + off[b] for m, b in mid]).to(dev)
    mslots = torch.cat([w.slots_of(b, m) for m, b in mid]).to(dev)
    ik.int4_kv_write(w.key[midx], w.value[midx], mslots, cache, signs)
    idx_n, slots_n = w.token_set("new")
    kn, vn, sn = w.key[idx_n.to(dev)].contiguous(), w.value[idx_n.to(dev)].contiguous(), slots_n.to(dev)
    ns = ik.int4kv_decode_num_segments(w.num_seqs, w.num_kv_heads, w.max_seqlen_k)
    segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size, dev) if ns > 1 else \
        (None, None, None)
    cu, su, bt = w.cu_seqlens_q().to(dev), w.seqused_k().to(dev), w.block_table.to(dev)
    out = torch.empty_like(w.query)
    sstep = lambda: ik.int4_decode_step(kn, vn, sn, w.query, cache, cu, su, 1, w.max_seqlen_k,  # noqa: E731
                                        bt, w.softmax_scale, signs, out=out, num_segments=ns,
                                        segm_output=segs[0], segm_max=segs[1],
                                        segm_expsum=segs[2])
    for _ in range(20):
        sstep()
    us = _graph_us(sstep, 20)
    rows["serving_standin"] = {
        "workload": f"{w.num_seqs} seqs: {w.num_seqs * P} prompt tokens written, then one decode "
                    f"step each at contexts {min(w.kv_lens)}..{max(w.kv_lens)} "
                    f"({sum(w.kv_lens)} keys), 32 q / 8 KV heads, d 128",
        "prompt_write_us": round(pw_us, 2),
        "prompt_write_tokens_per_s": round(w.num_seqs * P / pw_us * 1e6, 1),
        "num_segments": ns, "decode_step_us": round(us, 2),
        "timing": "prompt write: 10 back-to-back calls between events, per call; decode step: "
                  "20 steps replayed from one HIP graph, per step",
        "kv_GBps": round(w.kv_bytes_attended() / us / 1e3, 1)}
    del w, cache, sstep, kp, vp

    w = wl.llama3_8b_decode(device=dev)
    # its bulk cache fill (262144 tokens) and a decode step's write (64 tokens)
    cache = ik.empty_cache(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)
    _, slots_all = w.token_set("all")
    slots_all = slots_all.to(dev)
    signs = w.signs.to(dev)
    fill = lambda: ik.int4_kv_write(w.key, w.value, slots_all, cache, signs)  # noqa: E731
    for _ in range(2):
        fill()
    fill_us = _median_event_us(fill, 3)
    idx_new, slots_new = w.token_set("new")
    kn, vn = w.key[idx_new.to(dev)].contiguous(), w.value[idx_new.to(dev)].contiguous()
    slots_new = slots_new.to(dev)
    step_write = lambda: ik.int4_kv_write(kn, vn, slots_new, cache, signs)  # noqa: E731
    for _ in range(3):
        step_write()
    # 20 writes in one HIP graph: a launch this small is otherwise timed at the
    # host's call rate, not the GPU's
    g20 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g20):
        for _ in range(20):
            step_write()
    g20.replay()
    step_write_us = _median_event_us(g20.replay, 3) / 20
    T = w.key.shape[0]
    rows["llama3_8b_write"] = {
        "workload": "bulk fill of 262144 tokens (64 x 4096, 8 KV heads, d 128, bf16) and one "
                    "decode step's write of 64 tokens",
        "bulk_us": round(fill_us, 1), "bulk_tokens_per_s": round(T / fill_us * 1e6, 1),
        "bulk_GBps": round(w.write_bytes("all") / fill_us / 1e3, 1),
        "step_64_tokens_us": round(step_write_us, 2),
        "step_64_tokens_timing": "20 writes replayed from one HIP graph, per write"}
    del cache, fill, step_write, g20
    # the INT8 per-token-head mode's bulk fill of the same tokens (rows of d + 4 bytes)
    cache8 = ik.empty_cache_int8(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)
    fill8 = lambda: ik.int8_kv_write(w.key, w.value, slots_all, cache8)  # noqa: E731
    for _ in range(2):
        fill8()
    fill8_us = _median_event_us(fill8, 3)
    bytes8 = T * w.num_kv_heads * 2 * (2 * w.head_size + (w.head_size + 4)) + 8 * T
    rows["llama3_8b_write_int8"] = {
        "workload": "INT8 per-token-head bulk fill of the same 262144 tokens (rows of 132 bytes)",
        "bulk_us": round(fill8_us, 1), "bulk_tokens_per_s": round(T / fill8_us * 1e6, 1),
        "bulk_GBps": round(bytes8 / fill8_us / 1e3, 1)}
    del cache8, fill8
    # the INT2 Lloyd-Max mode's bulk fill (rows of d / 4 + 4 bytes, same rotation)
    sg = w.signs.to(dev)
    cache2 = ik.empty_cache_int2(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)
    fill2 = lambda: ik.int2_kv_write(w.key, w.value, slots_all, cache2, sg)  # noqa: E731
    for _ in range(2):
        fill2()
    fill2_us = _median_event_us(fill2, 3)
    bytes2 = T * w.num_kv_heads * 2 * (2 * w.head_size + (w.head_size // 4 + 4)) + 8 * T
    rows["llama3_8b_write_int2"] = {
        "workload": "INT2 Lloyd-Max bulk fill of the same 262144 tokens (rows of 36 bytes)",
        "bulk_us": round(fill2_us, 1), "bulk_tokens_per_s": round(T / fill2_us * 1e6, 1),
        "bulk_GBps": round(bytes2 / fill2_us / 1e3, 1)}
    del cache2, fill2
    best = None
    for ns in (1, 2, 4, 8):
        call = _attention_setup(w, dev, ns, ncaches=2)
        for _ in range(3):
            call()
        us_plain = _median_event_us(call, 20)
        us = _graph_us(call, 20)
        if best is None or us < best[1]:
            best = (ns, us, us_plain)
        del call
    kv = w.kv_bytes_attended()
    rows["llama3_8b_decode"] = {
        "workload": "64 seqs x 4096 tokens, 32 q / 8 KV heads, d 128 (outlier K channels)",
        "num_segments": best[0],
        "num_segments_library_choice": ik.int4kv_decode_num_segments(w.num_seqs, w.num_kv_heads,
                                                                     w.max_seqlen_k),
        "us": round(best[1], 2), "us_plain_calls": round(best[2], 2),
        "timing": "us: 20 calls (two caches alternating) replayed from one HIP graph, per call "
                  "(GPU time: back-to-back plain calls from Python are bound by the host's "
                  "call rate at this size)",
        "GBps": round(kv / best[1] / 1e3, 1), "hbm_frac": round(kv / best[1] / 1e3 / HBM_PEAK_GBS, 4)}

    # the same batch over the INT8 per-token-head cache (rows of 132 bytes); its
    # workgroups hold 4 KV heads, so half the INT4 split count fills the GPU
    _, slots8 = w.token_set("all")
    c8 = [ik.empty_cache_int8(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)]
    ik.int8_kv_write(w.key, w.value, slots8.to(dev), c8[0])
    c8.append(c8[0].clone())
    cu, su, bt = w.cu_seqlens_q().to(dev), w.seqused_k().to(dev), w.block_table.to(dev)
    out8 = torch.empty_like(w.query)
    st8 = {"i": 0}
    best8 = None
    for ns8 in (1, 2, 4):
        segs8 = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns8, w.head_size, dev) \
            if ns8 > 1 else (None, None, None)

        def call8():
            c = c8[st8["i"] % 2]
            st8["i"] += 1
            ik.int8_paged_attention(w.query, c, cu, su, 1, w.max_seqlen_k, bt, w.softmax_scale,
                                    out=out8, num_segments=ns8, segm_output=segs8[0],
                                    segm_max=segs8[1], segm_expsum=segs8[2])
        for _ in range(3):
            call8()
        us8 = _graph_us(call8, 20)
        if best8 is None or us8 < best8[1]:
            best8 = (ns8, us8)
    ns8, us8 = best8
    kv8 = sum(w.kv_lens) * w.num_kv_heads * 2 * (w.head_size + 4)
    rows["llama3_8b_decode_int8"] = {
        "workload": "the same 64 x 4096 batch over the INT8 per-token-head cache (132-byte rows)",
        "num_segments": ns8, "us": round(us8, 2),
        "num_segments_library_choice": ik.int8kv_decode_num_segments(w.num_seqs, w.num_kv_heads,
                                                                     w.max_seqlen_k),
        "timing": "20 calls (two caches alternating) replayed from one HIP graph, per call",
        "GBps": round(kv8 / us8 / 1e3, 1), "hbm_frac": round(kv8 / us8 / 1e3 / HBM_PEAK_GBS, 4),
        "kv_bytes_vs_int4": round(kv8 / kv, 3)}
    del c8

    # ... and over the INT2 Lloyd-Max cache (36-byte rows, same rotation and
    # split rule as INT4)
    c2 = [ik.empty_cache_int2(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)]
    ik.int2_kv_write(w.key, w.value, slots8.to(dev), c2[0], sg)
    c2.append(c2[0].clone())
    st2 = {"i": 0}
    best2 = None
    for ns2 in (2, 4, 8):
        segs2 = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns2, w.head_size, dev)

        def call2():
            c = c2[st2["i"] % 2]
            st2["i"] += 1
            ik.int2_paged_attention(w.query, c, cu, su, 1, w.max_seqlen_k, bt, w.softmax_scale, sg,
                                    out=out8, num_segments=ns2, segm_output=segs2[0],
                                    segm_max=segs2[1], segm_expsum=segs2[2])
        for _ in range(3):
            call2()
        us2 = _graph_us(call2, 20)
        if best2 is None or us2 < best2[1]:
            best2 = (ns2, us2)
    ns2, us2 = best2
    kv2 = sum(w.kv_lens) * w.num_kv_heads * 2 * (w.head_size // 4 + 4)
    rows["llama3_8b_decode_int2"] = {
        "workload": "the same 64 x 4096 batch over the INT2 Lloyd-Max cache (36-byte rows)",
        "num_segments": ns2, "us": round(us2, 2),
        "num_segments_library_choice": ik.int4kv_decode_num_segments(w.num_seqs, w.num_kv_heads,
                                                                     w.max_seqlen_k),
        "timing": "20 calls (two caches alternating) replayed from one HIP graph, per call",
        "GBps": round(kv2 / us2 / 1e3, 1), "hbm_frac": round(kv2 / us2 / 1e3 / HBM_PEAK_GBS, 4),
        "kv_bytes_vs_int4": round(kv2 / kv, 3)}
    return rows


def _first_sequences(w, n):
    """The first n sequences of a workload as a workload of their own (same
    cache ids): their K/V tokens, query rows and block-table rows."""
    off = w.token_offsets()
    cuq = w.cu_seqlens_q().tolist()
    dev = w.key.device
    return wl.Workload(w.name + f" first {n}", w.dtype, w.num_q_heads, w.num_kv_heads,
                       w.head_size, w.num_blocks, w.kv_lens[:n], w.query_lens[:n],
                       w.write_lens[:n], w.block_table[:n].clone(), w.key[:off[n]],
                       w.value[:off[n]], w.query[:cuq[n]], w.signs)


def _oracle_case(w, which_write="all"):
    """Host inputs of one workload for the oracle: raw bits, slots, metadata."""
    idx, slots = w.token_set(which_write)
    dev_idx = idx.to(w.key.device)
    return dict(kb=wl.bits16(w.key[dev_idx]), vb=wl.bits16(w.value[dev_idx]),
                qb=wl.bits16(w.query), slots=slots.numpy(), T=int(idx.numel()),
                dt="bf16" if w.dtype == torch.bfloat16 else "f16",
                cu=w.cu_seqlens_q().numpy(), su=w.seqused_k().numpy(),
                bt=w.block_table.numpy(), signs=w.signs.numpy(), w=w)


def _oracle_times(oracle, c, reps):
    """Median of `reps` runs of the oracle's write (all tokens of the case) and of
    its plain attention, seconds."""
    w = c["w"]
    tw, ta = [], []
    for _ in range(reps):
        cache = np.zeros(oracle.cache_shape(w.num_blocks, 16, w.num_kv_heads, w.head_size),
                         np.uint8)
        t0 = time.perf_counter()
        oracle.kv_write(c["kb"], c["vb"], c["dt"], c["slots"], cache, c["signs"])
        tw.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        oracle.attention_plain(c["qb"], c["dt"], cache, c["cu"], c["su"], c["bt"],
                               w.softmax_scale, c["signs"], w.num_q_heads)
        ta.append(time.perf_counter() - t0)
    return sorted(tw)[len(tw) // 2], sorted(ta)[len(ta) // 2]


def cpu_baseline(b, dev):
    """The oracle (plain C: fp32 encoding steps, textbook fp64 attention over the
    decoded cache) timed on this host: the long-context workload on one core
    (a bounded sample) and with OpenMP on every core this process may use
    (the whole workload), plus every other configuration with OpenMP.
    Median of three runs each; host inputs already in memory."""
    import oracle
    oracle._load()
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    omp = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores)))
    w = b["w"]
    key, value, _ = b["bulk"]
    full = dict(kb=wl.bits16(key), vb=wl.bits16(value), qb=wl.bits16(w.query),
                slots=w.token_set("all")[1].numpy(), dt="bf16", cu=w.cu_seqlens_q().numpy(),
                su=w.seqused_k().numpy(), bt=w.block_table.numpy(), signs=w.signs.numpy(), w=w)
    kv = w.kv_bytes_attended()
    # one core: sequence 0 of the four (131072 keys), written and attended
    one = wl.Workload(w.name + " seq 0", w.dtype, w.num_q_heads, w.num_kv_heads, w.head_size,
                      w.num_blocks, w.kv_lens[:1], w.query_lens[:1], w.write_lens[:1],
                      w.block_table[:1].clone(), key[:w.kv_lens[0]], value[:w.kv_lens[0]],
                      w.query[:1], w.signs)
    c1 = _oracle_case(one)
    oracle.set_num_threads(1)
    tw1, ta1 = _oracle_times(oracle, c1, 3)
    kv1 = one.kv_bytes_attended()
    oracle.set_num_threads(omp)
    twn, tan = _oracle_times(oracle, full, 3)
    res = {"value": round(kv / tan / 1e9, 4), "unit": "GB/s", "cores": omp, "kind": "oracle",
           "sample": f"the whole long-context workload (4 x 131072 keys, 8 KV heads, 64 query "
                     f"heads) on {omp} OpenMP threads: plain fp64 attention {tan:.3f} s, its "
                     f"cache write of {key.shape[0]} tokens {twn:.3f} s (median of 3)",
           "write_tokens_per_s": round(key.shape[0] / twn, 1),
           "single_core": {"value": round(kv1 / ta1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                           "sample": f"sequence 0 of the workload (131072 keys): attention "
                                     f"{ta1:.3f} s, write {tw1:.3f} s (median of 3)",
                           "write_tokens_per_s": round(one.kv_lens[0] / tw1, 1)},
           "host_cpus": cores}
    # the other configurations, OpenMP, median of 3 (the chunked-prefill mix on a
    # sample of its first 4 sequences: its plain attention is the longest)
    per = {}
    for name, wk in (("tiny_causal", wl.tiny()), ("gqa_decode", wl.gqa_decode()),
                     ("llama3_8b_decode", wl.llama3_8b_decode(device=dev)),
                     ("chunked_prefill_d128_first4",
                      _first_sequences(wl.chunked_prefill(device=dev), 4))):
        c = _oracle_case(wk)
        tw, ta = _oracle_times(oracle, c, 3)
        per[name] = {"write_tokens": c["T"], "write_s": round(tw, 4),
                     "write_tokens_per_s": round(c["T"] / tw, 1),
                     "attention_s": round(ta, 4),
                     "attention_kv_GBps": round(wk.kv_bytes_attended() / ta / 1e9, 4)}
        del c, wk
    res["configs"] = per
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-rows", action="store_true",
                    help="skip the prefill and Llama-3-shaped decode measurements")
    ap.add_argument("--only-other-rows", action="store_true",
                    help="only the prefill and Llama-3-shaped decode measurements (for profiling)")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of the library calls instead of plain calls")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time the step as int4_kv_write + int4_paged_attention (two calls)")
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
    if args.only_other_rows:
        print(json.dumps({"other_rows": other_rows(dev)}), flush=True)
        return
    nbufs = 2  # 2 x 570 MB > 256 MB Infinity Cache
    bufs = build_buffers(nbufs, dev)
    log("caches filled")
    w = bufs[0]["w"]
    kv_bytes = w.kv_bytes_attended()

    step_fn = step_separate if args.separate_calls else step
    if args.graph:
        graphs = [capture(lambda b=b: step_fn(b)) for b in bufs]
        attn_graphs = [capture(lambda b=b: attend(b)) for b in bufs]
        check_replay(bufs, attn_graphs)
        run = [g.replay for g in graphs]
        run_attn = [g.replay for g in attn_graphs]
    else:
        run = [lambda b=b: step_fn(b) for b in bufs]
        run_attn = [lambda b=b: attend(b) for b in bufs]

    settled = settle(run, nbufs)
    for i in range(args.warmup):
        run[i % nbufs]()
    torch.cuda.synchronize()
    wall, step_ev_ms = timed_block(run, nbufs, args.steps)
    ms_per_step = wall * 1e3 / args.steps
    # per-step statistics: the same steps again, an event after each
    _, step_ms = timed_calls(run, nbufs, args.steps)

    # the attention call alone (decode + segment reduction), warmed up the same
    # way; HIP events on the launch stream before the first and after the last
    for i in range(args.warmup):
        run_attn[i % nbufs]()
    attn_wall, attn_ev_ms = timed_block(run_attn, nbufs, args.steps)
    attn_s = attn_ev_ms / 1e3 / args.steps
    _, attn_ms = timed_calls(run_attn, nbufs, args.steps)

    gather_us = gather_only(bufs, args.steps)
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step; attention {attn_s * 1e6:.2f} us; "
        f"its gather alone {gather_us:.2f} us")
    wr_tps, wr_t, wr_T = measure_bulk_write(bufs[0])
    bk, bv, bslots = bufs[0]["bulk"]
    wr_read = bk.numel() * bk.element_size() + bv.numel() * bv.element_size() + bslots.numel() * 8
    wr_written = w.write_bytes("all") - wr_read  # write_bytes counts the inputs read too
    st_t, st_r, st_w = measure_stream_ceiling(wr_read, wr_written)
    value = kv_bytes / (ms_per_step / 1e3) / 1e9
    achieved = kv_bytes / attn_s / 1e9
    traffic = _traffic_from_profiles(_kernel_hash())
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8 mfma (scores) + f16 mfma (P.V), f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "long-context decode: 4 seqs x 131072 tokens, 64 q / 8 KV heads, "
                               "head_size 128, bf16 K/V/Q N(0,1), block_size 16, split-K 64 "
                               "segments + segment reduction; step = write 4 new tokens + decode",
                   "step_call": ("int4_kv_write + int4_paged_attention" if args.separate_calls
                                 else "int4_decode_step (write fused into the decode launch)"),
                   "global_batch": 4, "seq_len": 131072, "parallelism": "none (1 GPU)",
                   "launch": "hip graph replay" if args.graph else "plain calls",
                   "settle": settled},
        "timed_region_event_us_per_step": round(step_ev_ms * 1e3 / args.steps, 2),
        "step_events": call_stats(step_ms) if step_ms else None,
        "attention_call_events": call_stats(attn_ms) if attn_ms else None,
        "per_call_events_note": "step_events / attention_call_events: a second pass of the same "
                                "K calls with an event after each (those events cost the calls "
                                "2-3 us each); ms_per_step and roofline come from passes with "
                                "events only before the first and after the last call",
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "num_segments_library_choice": ik.int4kv_decode_num_segments(w.num_seqs, w.num_kv_heads,
                                                                     w.max_seqlen_k),
        "write_tokens_per_s": round(wr_tps, 1),
        "write_bulk": {"tokens": wr_T, "seconds": wr_t,
                       "bytes_read": wr_read, "bytes_written": wr_written,
                       "GB_per_s": round(wr_written / wr_t / 1e9, 1),
                       "read_plus_write_GB_per_s": round((wr_read + wr_written) / wr_t / 1e9, 1),
                       "stream_same_mix": {
                           "seconds": st_t, "bytes_read": st_r, "bytes_written": st_w,
                           "read_plus_write_GB_per_s": round((st_r + st_w) / st_t / 1e9, 1),
                           "write_time_over_stream_time": round(wr_t / st_t, 4)}},
        "roofline": {"kernel": "decode_lds_kernel + reduce_wave_kernel (one int4_paged_attention call)",
                     "timing": "HIP events on the launch stream before the first and after the "
                               "last of K back-to-back attention calls, / K (decode kernel, "
                               "segment reduction, the dispatch gaps)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": kv_bytes,
                     "avg_launch_us": round(attn_s * 1e6, 2),
                     "gather_only": {
                         "call": "int4kv_stream_blocks: the attention call's block gather alone "
                                 "(same blocks, order, workgroups and LDS ring, nothing "
                                 "computed), timed like the attention call",
                         "us": round(gather_us, 2),
                         "GB_per_s": round(kv_bytes / gather_us / 1e3, 1),
                         "frac_of_peak": round(kv_bytes / gather_us / 1e3 / HBM_PEAK_GBS, 4),
                         "attention_call_over_gather": round(attn_s * 1e6 / gather_us, 4)}},
    }
    if not args.no_other_rows:
        res["other_rows"] = other_rows(dev)
        log("other rows measured")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(bufs[0], dev)
        log("oracle baseline timed")
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

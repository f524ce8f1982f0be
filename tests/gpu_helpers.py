"""Shared set-up for the GPU parity tests: drive the HIP library and the CPU
oracle from the same seeded workload, never feeding one's output to the other."""
import numpy as np
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl

SENTINEL = 0xA5
ATOL, RTOL = 2e-3, 1e-2  # attention parity bound, fp32 accumulation


def dt_name(w):
    return "bf16" if w.dtype == torch.bfloat16 else "f16"


def header(msg):
    print(f"[gpu-case] {msg}", flush=True)


def to_dev(w, dev="cuda"):
    """Inputs of a workload on the GPU (generation happened elsewhere)."""
    return dict(key=w.key.to(dev), value=w.value.to(dev), query=w.query.to(dev),
                signs=w.signs.to(dev), block_table=w.block_table.to(dev),
                cu=w.cu_seqlens_q().to(dev), su=w.seqused_k().to(dev))


def gpu_cache(w, dev="cuda", fill=SENTINEL):
    c = ik.empty_cache(w.num_blocks, w.num_kv_heads, w.head_size, device=dev)
    c.fill_(fill)
    return c


def gpu_write(w, t, cache, which="all"):
    idx, slots = w.token_set(which)
    if idx.numel() == 0:
        return
    dev = cache.device
    idx_d = idx.to(dev)
    ik.int4_kv_write(t["key"][idx_d], t["value"][idx_d], slots.to(dev), cache, t["signs"])


def oracle_cache(orc, w, which="all", fill=SENTINEL, token_subset=None):
    cache = np.full(orc.cache_shape(w.num_blocks, w.block_size, w.num_kv_heads, w.head_size),
                    fill, np.uint8)
    idx, slots = w.token_set(which)
    if token_subset is not None:
        keep = torch.isin(idx, token_subset)
        idx, slots = idx[keep], slots[keep]
    orc.kv_write(wl.bits16(w.key[idx.to(w.key.device)]), wl.bits16(w.value[idx.to(w.key.device)]),
                 dt_name(w), slots.numpy(), cache, w.signs.numpy())
    return cache


def gpu_attention(w, t, cache, num_segments=1, query=None, window=0, softcap=0.0):
    q = t["query"] if query is None else query
    segs = (None, None, None)
    if num_segments > 1 and w.max_seqlen_q == 1:
        segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, num_segments, w.head_size,
                                  device=cache.device)
    return ik.int4_paged_attention(q, cache, t["cu"], t["su"], w.max_seqlen_q, w.max_seqlen_k,
                                   t["block_table"], w.softmax_scale, t["signs"],
                                   num_segments=num_segments, segm_output=segs[0],
                                   segm_max=segs[1], segm_expsum=segs[2], sliding_window=window,
                                   softcap=softcap)


def oracle_attention(orc, w, cache, window=0, softcap=0.0):
    return orc.attention_plain(wl.bits16(w.query), dt_name(w), cache, w.cu_seqlens_q().numpy(),
                               w.seqused_k().numpy(), w.block_table.numpy(), w.softmax_scale,
                               w.signs.numpy(), w.num_q_heads, window=window, softcap=softcap)


def assert_attention_close(got, ref, what="", atol_scale=1.0):
    """|got - ref| <= 2e-3 * atol_scale + 1e-2 |ref| elementwise.

    ``atol_scale`` only ever shrinks the absolute term (inputs scaled down by
    c < 1 pass c, so the bound keeps its meaning for outputs of size c); it
    never widens it.  Prints the worst err/bound ratio, and checks that the
    bound bites: an all-zero output must fail it wherever the reference is
    not itself all zero."""
    assert 0.0 < atol_scale <= 1.0, "the absolute term is never widened"
    g = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(g - ref)
    atol = ATOL * atol_scale
    bound = atol + RTOL * np.abs(ref)
    ratio = float((err / bound).max()) if err.size else 0.0
    print(f"[parity] {what}: worst err/bound {ratio:.3g}, max err {err.max() if err.size else 0:.3g}",
          flush=True)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside "
                           f"{atol:.3g} + 1e-2|ref|; worst err/bound {ratio:.3g} at "
                           f"{np.unravel_index((err / bound).argmax(), err.shape)}; "
                           f"max err {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}")
    if np.any(ref != 0.0):
        assert np.any(np.abs(ref) > bound), f"{what}: an all-zero output would pass this bound"
    return float(err.max()) if err.size else 0.0


def sub_workload(w, seqs):
    """The sequences ``seqs`` of ``w`` as a batch of their own (same cache ids)."""
    off = w.token_offsets()
    cuq = w.cu_seqlens_q().tolist()
    kidx = torch.cat([torch.arange(off[b], off[b + 1]) for b in seqs])
    qidx = torch.cat([torch.arange(cuq[b], cuq[b + 1]) for b in seqs])
    return wl.Workload(w.name + f" seqs {seqs}", w.dtype, w.num_q_heads, w.num_kv_heads,
                       w.head_size, w.num_blocks, [w.kv_lens[b] for b in seqs],
                       [w.query_lens[b] for b in seqs], [w.write_lens[b] for b in seqs],
                       w.block_table[seqs].clone(), w.key[kidx.to(w.key.device)],
                       w.value[kidx.to(w.key.device)], w.query[qidx.to(w.key.device)], w.signs)

"""GPU parity of prefill / mixed-batch attention (query lengths > 1).

Oracle: textbook causal attention in fp64 over the oracle's own encoding of the
raw K/V.  Bound |gpu - ref| <= 2e-3 + 1e-2 |ref|."""
import numpy as np
import pytest
import torch

from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import (assert_attention_close, gpu_attention, gpu_cache, gpu_write, header,
                               oracle_attention, oracle_cache, to_dev)

pytestmark = pytest.mark.gpu


def _run(oracle_mod, w, atol_scale=1.0):
    header(f"prefill {w.name}")
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    out = gpu_attention(w, t, c)
    torch.cuda.synchronize()
    ref = oracle_attention(oracle_mod, w, oracle_cache(oracle_mod, w, "all"))
    assert_attention_close(out, ref, w.name, atol_scale)
    return out


MIX = [(5, 48), (16, 16), (1, 100), (33, 33), (64, 200), (7, 301), (2, 2), (1, 1)]


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_prefill_mixed_lengths(oracle_mod, G, d):
    hkv = 2 if G <= 8 else 1
    w = wl.custom(MIX, G * hkv, hkv, d, dtype=torch.bfloat16, seed=100 + G + d, write_all=True,
                  extra_blocks=2)
    _run(oracle_mod, w)


@pytest.mark.parametrize("scale", [1e-3, 30.0])
@pytest.mark.parametrize("G,d", [(4, 128), (8, 64)])
def test_prefill_scaled_inputs(oracle_mod, scale, G, d):
    """fp16 inputs scaled down (tiny scales, subnormal-range f16 weights) and
    up (logits of order 10^3: the query's hi + lo split must carry them)."""
    w = wl.custom([(40, 120), (9, 300)], G * 2, 2, d, dtype=torch.float16, seed=11 + G + d,
                  write_all=True, scale=scale)
    _run(oracle_mod, w, atol_scale=min(1.0, scale))


def test_prefill_fp16_long_prompt(oracle_mod):
    w = wl.custom([(150, 1000), (97, 97)], 8, 2, 128, dtype=torch.float16, seed=7, write_all=True)
    _run(oracle_mod, w)


def test_prefill_last_row_matches_decode(oracle_mod):
    """The last query row of a prefill equals a decode at the same position."""
    w = wl.custom([(40, 390)], 32, 8, 128, seed=9, write_all=True)
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    pre = gpu_attention(w, t, c)
    dq = wl.Workload(w.name, w.dtype, 32, 8, 128, w.num_blocks, [390], [1], [1], w.block_table,
                     w.key, w.value, w.query[-1:], w.signs)
    td = to_dev(dq)
    dec = gpu_attention(dq, td, c, 4)
    torch.cuda.synchronize()
    ref = oracle_attention(oracle_mod, dq, oracle_cache(oracle_mod, dq, "all"))
    assert_attention_close(pre[-1:], ref, "prefill last row")
    assert_attention_close(dec, ref, "decode")


@pytest.mark.parametrize("d", [128, 64])
def test_chunked_prefill_full_size_sampled(oracle_mod, d):
    """32 sequences, query lengths log-uniform in [1, 512], contexts in
    [512, 16384]: the whole mixed batch on the GPU; 12 sampled (sequence, query
    row) pairs checked against the oracle, which evaluates each sampled row as a
    decode at that row's position over its own encoding of the raw K/V."""
    w = wl.chunked_prefill(device="cuda", head_size=d)
    header(f"chunked prefill full size d={d}: {sum(w.query_lens)} query tokens")
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    out = gpu_attention(w, t, c)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(d)
    off = w.token_offsets()
    cuq = w.cu_seqlens_q().tolist()
    for b in torch.randperm(w.num_seqs, generator=g)[:12].tolist():
        ql, L = w.query_lens[b], w.kv_lens[b]
        i = int(torch.randint(0, ql, (1,), generator=g))
        pos = L - ql + i
        kidx = torch.arange(off[b], off[b] + pos + 1).to(w.key.device)
        sub = wl.Workload("row", w.dtype, w.num_q_heads, w.num_kv_heads, d, w.num_blocks,
                          [pos + 1], [1], [1], w.block_table[[b]].clone(), w.key[kidx],
                          w.value[kidx], w.query[cuq[b] + i:cuq[b] + i + 1], w.signs)
        ref = oracle_attention(oracle_mod, sub, oracle_cache(oracle_mod, sub, "all"))
        assert_attention_close(out[cuq[b] + i:cuq[b] + i + 1], ref, f"seq {b} row {i}")


def test_prefill_many_groups_long_context(oracle_mod):
    """The workgroups' launch ranking beyond one pass of its 512 threads: 163
    sequences (652 (sequence, query tile) groups at 32 q / 8 KV heads, many of
    them empty), and contexts past 1,022 key tiles, where the ranking scales
    the tile counts into its buckets; every output row checked."""
    g = torch.Generator().manual_seed(77)
    lens = []
    for _ in range(160):
        q = int(torch.randint(1, 101, (1,), generator=g))
        lens.append((q, q + int(torch.randint(0, 201, (1,), generator=g))))
    lens += [(2, 40000), (33, 36000), (128, 128)]
    w = wl.custom(lens, 32, 8, 128, dtype=torch.bfloat16, seed=78, write_all=True)
    _run(oracle_mod, w)


def test_prefill_batch_invariance():
    """A sequence's prefill output does not depend on the rest of the batch or
    on the launch order: the chunked-prefill mix (3,328 workgroups, ranked
    longest first) against four of its sequences run alone (few workgroups,
    launched in index order), bit for bit."""
    from tests.gpu_helpers import sub_workload
    w = wl.chunked_prefill(device="cuda")
    header("prefill batch invariance")
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    out = gpu_attention(w, t, c)
    cuq = w.cu_seqlens_q().tolist()
    for b in (0, 4, 7, 19):  # (query lengths 20, 372, 114, 4: all prefill rows)
        ws = sub_workload(w, [b])
        ts = to_dev(ws)
        o1 = gpu_attention(ws, ts, c)  # same cache ids, one sequence
        torch.cuda.synchronize()
        assert torch.equal(o1, out[cuq[b]:cuq[b + 1]]), f"sequence {b}"

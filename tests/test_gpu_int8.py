"""GPU parity of the INT8 per-token-head mode: the cache write (codes and
scale words bit for bit against the oracle over the whole cache buffer,
sentinel bytes included), and decode and prefill attention over that cache
(|gpu - ref| <= 2e-3 + 1e-2 |ref| against the oracle's fp64 attention)."""
import random

import numpy as np
import pytest
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import SENTINEL, header

pytestmark = pytest.mark.gpu


def _write_both(oracle_mod, key, value, slots, nb, hkv, d, key_dev=None, value_dev=None):
    c = torch.full(ik.cache_shape_int8(nb, hkv, d), SENTINEL, dtype=torch.uint8, device="cuda")
    ik.int8_kv_write(key.cuda() if key_dev is None else key_dev,
                     value.cuda() if value_dev is None else value_dev, slots.cuda(), c)
    ref = np.full(oracle_mod.cache_shape_int8(nb, 16, hkv, d), SENTINEL, np.uint8)
    oracle_mod.kv_write_int8(wl.bits16(key), wl.bits16(value),
                             "bf16" if key.dtype == torch.bfloat16 else "f16", slots.numpy(), ref)
    torch.cuda.synchronize()
    return c.cpu().numpy(), ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hkv", [1, 4, 8])
@pytest.mark.parametrize("T", [1, 7, 42, 1000])
def test_int8_write_bit_exact(oracle_mod, T, hkv, d, dtype):
    header(f"int8 write T={T} hkv={hkv} d={d} {dtype}")
    random.seed(T + hkv + d)
    g = torch.Generator().manual_seed(T * 100 + hkv * 10 + d)
    nb = (T + 15) // 16 + 4
    slots = torch.tensor(random.sample(range(nb * 16), T), dtype=torch.int64)
    key = (2.0 * torch.randn((T, hkv, d), generator=g)).to(dtype)
    value = torch.randn((T, hkv, d), generator=g).to(dtype)
    got, ref = _write_both(oracle_mod, key, value, slots, nb, hkv, d)
    assert np.array_equal(got, ref)


def test_int8_write_ties_zero_rows_and_skips(oracle_mod):
    """Rows whose scaled values sit on exact .5 ties (absmax 127 gives scale 1),
    all-zero rows (the 1e-6 floor) and negative slots (nothing written)."""
    header("int8 write ties / zero rows / skips")
    d, T = 128, 48
    base = torch.arange(-63.5, 64.5, 1.0)[:d]  # halves: ties at scale 1
    key = torch.stack([base.clone() for _ in range(T)]).view(T, 1, d)
    key[:, 0, 0] = 127.0
    key[1::3] = 0.0
    value = -key
    slots = torch.arange(T, dtype=torch.int64) * 2
    slots[::5] = -1
    for dtype in (torch.bfloat16, torch.float16):
        got, ref = _write_both(oracle_mod, key.to(dtype), value.to(dtype), slots, 8, 1, d)
        assert np.array_equal(got, ref), dtype


def test_int8_write_strided_token_layout(oracle_mod):
    header("int8 write strided qkv")
    g = torch.Generator().manual_seed(12)
    T, hq, hkv, d = 37, 32, 8, 128
    qkv = torch.randn((T, hq + 2 * hkv, d), generator=g).to(torch.bfloat16)
    qkv_d = qkv.cuda()
    key, value = qkv[:, hq:hq + hkv], qkv[:, hq + hkv:]
    slots = torch.randperm(64 * 16, generator=g)[:T].to(torch.int64)
    got, ref = _write_both(oracle_mod, key.contiguous(), value.contiguous(), slots, 64, hkv, d,
                           key_dev=qkv_d[:, hq:hq + hkv], value_dev=qkv_d[:, hq + hkv:])
    assert np.array_equal(got, ref)


def test_int8_write_llama3_bulk_fill_sampled(oracle_mod):
    """64 x 4096 tokens, 8 KV heads, d 128, in the launch the benchmark times;
    3000 sampled tokens bit for bit, and every row written."""
    header("int8 write Llama-3-8B-shaped bulk fill (sampled)")
    w = wl.llama3_8b_decode(device="cuda")
    idx, slots = w.token_set("all")
    c = torch.full(ik.cache_shape_int8(w.num_blocks, 8, 128), SENTINEL, dtype=torch.uint8,
                   device="cuda")
    ik.int8_kv_write(w.key, w.value, slots.cuda(), c)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(2)
    pick = torch.randperm(idx.numel(), generator=g)[:3000]
    ref = np.full(oracle_mod.cache_shape_int8(w.num_blocks, 16, 8, 128), SENTINEL, np.uint8)
    oracle_mod.kv_write_int8(wl.bits16(w.key[pick.cuda()]), wl.bits16(w.value[pick.cuda()]),
                             "bf16", slots[pick].numpy(), ref)
    s = slots[pick]
    blk, off = (s // 16).numpy(), (s % 16).numpy()
    got = c.cpu().numpy()
    assert np.array_equal(got[blk, :, off], ref[blk, :, off])
    words = got[..., 128:132].copy().view("<u4")[..., 0]
    assert ((words & 0x7F800000) != 0x7F800000).all() and (words != 0xA5A5A5A5).all()


# ---- decode attention over the INT8 cache

from tests.gpu_helpers import assert_attention_close, sub_workload, to_dev  # noqa: E402


def _int8_cache(oracle_mod, w, t):
    c = torch.full(ik.cache_shape_int8(w.num_blocks, w.num_kv_heads, w.head_size), SENTINEL,
                   dtype=torch.uint8, device="cuda")
    idx, slots = w.token_set("all")
    ik.int8_kv_write(t["key"][idx.cuda()], t["value"][idx.cuda()], slots.cuda(), c)
    ref = np.full(oracle_mod.cache_shape_int8(w.num_blocks, 16, w.num_kv_heads, w.head_size),
                  SENTINEL, np.uint8)
    oracle_mod.kv_write_int8(wl.bits16(w.key[idx.to(w.key.device)]),
                             wl.bits16(w.value[idx.to(w.key.device)]),
                             "bf16" if w.dtype == torch.bfloat16 else "f16", slots.numpy(), ref)
    return c, ref


def _attn8(w, t, c, ns=1, window=0, softcap=0.0):
    segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size) if ns > 1 else \
        (None, None, None)
    return ik.int8_paged_attention(t["query"], c, t["cu"], t["su"], w.max_seqlen_q, w.max_seqlen_k,
                                   t["block_table"], w.softmax_scale, num_segments=ns,
                                   segm_output=segs[0], segm_max=segs[1], segm_expsum=segs[2],
                                   sliding_window=window, softcap=softcap)


def _ref8(oracle_mod, w, ref_cache, window=0, softcap=0.0):
    return oracle_mod.attention_plain_int8(
        wl.bits16(w.query), "bf16" if w.dtype == torch.bfloat16 else "f16", ref_cache,
        w.cu_seqlens_q().numpy(), w.seqused_k().numpy(), w.block_table.numpy(), w.softmax_scale,
        w.num_q_heads, window=window, softcap=softcap)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_int8_decode_ragged_lengths(oracle_mod, G, d):
    lens = [(1, 1), (1, 15), (1, 16), (1, 17), (1, 33), (1, 100), (1, 517)]
    hkv = 4 if G <= 4 else 2
    w = wl.custom(lens, G * hkv, hkv, d, seed=G * 13 + d, write_all=True, extra_blocks=3)
    t = to_dev(w)
    c, ref_cache = _int8_cache(oracle_mod, w, t)
    assert np.array_equal(c.cpu().numpy(), ref_cache)
    ref = _ref8(oracle_mod, w, ref_cache)
    for ns in (1, 2, 5, 64):
        header(f"int8 decode G={G} d={d} NS={ns}")
        out = _attn8(w, t, c, ns)
        torch.cuda.synchronize()
        assert_attention_close(out, ref, f"int8 G={G} d={d} NS={ns}")


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (64, 8, 64), (8, 1, 128), (32, 16, 128)])
def test_int8_decode_heads_window_softcap_large_values(oracle_mod, hq, hkv, d):
    w = wl.custom([(1, 300), (1, 77), (1, 513), (1, 2000)], hq, hkv, d, seed=hq + hkv + d,
                  write_all=True, scale=3.0)
    t = to_dev(w)
    c, ref_cache = _int8_cache(oracle_mod, w, t)
    for window, cap in ((0, 0.0), (100, 0.0), (0, 5.0), (300, 30.0)):
        ref = _ref8(oracle_mod, w, ref_cache, window, cap)
        for ns in (1, 16):
            header(f"int8 decode {hq}/{hkv} d{d} window={window} cap={cap} NS={ns}")
            out = _attn8(w, t, c, ns, window, cap)
            torch.cuda.synchronize()
            assert_attention_close(out, ref, f"window {window} cap {cap} NS={ns}")
    w30 = wl.custom([(1, 300), (1, 77), (1, 513), (1, 160)] * 2, hq, hkv, d, seed=5 + hq,
                    write_all=True, scale=30.0, dtype=torch.float16)
    t30 = to_dev(w30)
    c30, ref30 = _int8_cache(oracle_mod, w30, t30)
    for ns in (1, 7):
        header(f"int8 decode large values {hq}/{hkv} d{d} NS={ns}")
        assert_attention_close(_attn8(w30, t30, c30, ns), _ref8(oracle_mod, w30, ref30),
                               f"large values NS={ns}")


def test_int8_decode_empty_and_zero_length(oracle_mod):
    w = wl.custom([(1, 40), (0, 20), (1, 0), (1, 9)], 8, 2, 128, seed=4, write_all=True)
    t = to_dev(w)
    c, ref_cache = _int8_cache(oracle_mod, w, t)
    ref = _ref8(oracle_mod, w, ref_cache)
    for ns in (1, 3):
        out = _attn8(w, t, c, ns)
        torch.cuda.synchronize()
        assert_attention_close(out, ref, f"NS={ns}")
        assert torch.all(out[1].float() == 0.0)


def test_int8_decode_llama3_full_size_sampled(oracle_mod):
    """64 x 4096, 32 q / 8 KV heads, in the launch the benchmark times (the
    library's split count); 3 sampled sequences against the oracle."""
    w = wl.llama3_8b_decode(device="cuda")
    ns = ik.int8kv_decode_num_segments(w.num_seqs, w.num_kv_heads, w.max_seqlen_k)
    header(f"int8 Llama-3-8B-shaped decode full size NS={ns}")
    t = to_dev(w)
    c = torch.empty(ik.cache_shape_int8(w.num_blocks, 8, 128), dtype=torch.uint8, device="cuda")
    idx, slots = w.token_set("all")
    ik.int8_kv_write(w.key, w.value, slots.cuda(), c)
    out = _attn8(w, t, c, ns)
    torch.cuda.synchronize()
    for seqs in ([0], [37], [63]):
        ws = sub_workload(w, seqs)
        ref_cache = np.zeros(oracle_mod.cache_shape_int8(ws.num_blocks, 16, 8, 128), np.uint8)
        i2, s2 = ws.token_set("all")
        oracle_mod.kv_write_int8(wl.bits16(ws.key[i2.to(ws.key.device)]),
                                 wl.bits16(ws.value[i2.to(ws.key.device)]), "bf16", s2.numpy(),
                                 ref_cache)
        assert_attention_close(out[seqs], _ref8(oracle_mod, ws, ref_cache), f"seq {seqs}")


# ---- prefill / mixed batches over the INT8 cache

MIX = [(5, 48), (16, 16), (1, 100), (33, 33), (64, 200), (7, 301), (2, 2), (1, 1)]


def _prefill8(oracle_mod, w, window=0, softcap=0.0, atol_scale=1.0):
    t = to_dev(w)
    c, ref_cache = _int8_cache(oracle_mod, w, t)
    out = _attn8(w, t, c, 1, window, softcap)
    torch.cuda.synchronize()
    assert_attention_close(out, _ref8(oracle_mod, w, ref_cache, window, softcap), w.name,
                           atol_scale)
    return out


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [64, 128])
def test_int8_prefill_mixed_lengths(oracle_mod, G, d):
    """Query lengths 1..64 over contexts 1..301 in one batch: ragged query
    tiles, tiles that end mid-block and single-token rows."""
    header(f"int8 prefill mixed G={G} d={d}")
    hkv = 2 if G <= 8 else 1
    w = wl.custom(MIX, G * hkv, hkv, d, seed=300 + G + d, write_all=True, extra_blocks=2)
    _prefill8(oracle_mod, w)


@pytest.mark.parametrize("hq,hkv,d,dtype", [(6, 3, 128, torch.float16), (32, 8, 64, torch.bfloat16)])
def test_int8_prefill_window_softcap(oracle_mod, hq, hkv, d, dtype):
    """Sliding windows shorter and longer than the query tile, soft caps, and a
    KV head count (3) that the decode kernel does not take."""
    w = wl.custom([(40, 120), (9, 300), (130, 130)], hq, hkv, d, dtype=dtype, seed=hq + d,
                  write_all=True, scale=2.0)
    for window, cap in ((0, 0.0), (17, 0.0), (100, 0.0), (0, 5.0), (50, 30.0)):
        header(f"int8 prefill {hq}/{hkv} d{d} window={window} cap={cap}")
        _prefill8(oracle_mod, w, window, cap)


@pytest.mark.parametrize("scale", [1e-3, 30.0])
def test_int8_prefill_scaled_inputs(oracle_mod, scale):
    header(f"int8 prefill scale {scale}")
    w = wl.custom([(40, 120), (9, 300)], 8, 2, 128, dtype=torch.float16, seed=17, write_all=True,
                  scale=scale)
    _prefill8(oracle_mod, w, atol_scale=min(1.0, scale))


def test_int8_prefill_empty_sequences_and_last_row_matches_decode(oracle_mod):
    """Zero-length queries and contexts inside a prefill batch write nothing
    to their rows; the last query row of a prefill equals the decode of the
    same token."""
    header("int8 prefill empty sequences / last row vs decode")
    w = wl.custom([(30, 60), (0, 20), (3, 3), (40, 390)], 32, 8, 128, seed=21, write_all=True)
    t = to_dev(w)
    c, ref_cache = _int8_cache(oracle_mod, w, t)
    pre = _attn8(w, t, c)
    ref = _ref8(oracle_mod, w, ref_cache)
    torch.cuda.synchronize()
    assert_attention_close(pre, ref, "prefill")
    last = sub_workload(w, [3])
    dq = wl.Workload("last row", w.dtype, 32, 8, 128, w.num_blocks, [390], [1], [1],
                     last.block_table, last.key, last.value, last.query[-1:], w.signs)
    dec = _attn8(dq, to_dev(dq), c, 4)
    torch.cuda.synchronize()
    assert_attention_close(dec, ref[-1:], "decode of the last row")


def test_int8_chunked_prefill_full_size_sampled(oracle_mod):
    """The 32-sequence chunked-prefill mix (query lengths log-uniform in
    [1, 512], contexts in [512, 16384], 32 q / 8 KV heads, d 128) in one
    launch; 10 sampled (sequence, query row) pairs against the oracle, each
    evaluated as a decode at that row's position."""
    w = wl.chunked_prefill(device="cuda")
    header(f"int8 chunked prefill full size: {sum(w.query_lens)} query tokens")
    t = to_dev(w)
    c = torch.empty(ik.cache_shape_int8(w.num_blocks, 8, 128), dtype=torch.uint8, device="cuda")
    idx, slots = w.token_set("all")
    ik.int8_kv_write(w.key, w.value, slots.cuda(), c)
    out = _attn8(w, t, c)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(8)
    off = w.token_offsets()
    cuq = w.cu_seqlens_q().tolist()
    for b in torch.randperm(w.num_seqs, generator=g)[:10].tolist():
        ql, L = w.query_lens[b], w.kv_lens[b]
        i = int(torch.randint(0, ql, (1,), generator=g))
        pos = L - ql + i
        kidx = torch.arange(off[b], off[b] + pos + 1).to(w.key.device)
        sub = wl.Workload("row", w.dtype, 32, 8, 128, w.num_blocks, [pos + 1], [1], [1],
                          w.block_table[[b]].clone(), w.key[kidx], w.value[kidx],
                          w.query[cuq[b] + i:cuq[b] + i + 1], w.signs)
        ref_cache = np.zeros(oracle_mod.cache_shape_int8(w.num_blocks, 16, 8, 128), np.uint8)
        i2, s2 = sub.token_set("all")
        oracle_mod.kv_write_int8(wl.bits16(sub.key[i2.to(sub.key.device)]),
                                 wl.bits16(sub.value[i2.to(sub.key.device)]), "bf16", s2.numpy(),
                                 ref_cache)
        assert_attention_close(out[cuq[b] + i:cuq[b] + i + 1], _ref8(oracle_mod, sub, ref_cache),
                               f"seq {b} row {i}")

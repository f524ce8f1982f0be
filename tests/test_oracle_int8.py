"""Pins of the oracle's INT8 per-token-head mode (rows of d int8 codes and an
fp32 scale, no rotation; readings R8-layout, R8-quant, R8-round, R8-deq):

  * the pages' INT8 worked example (tests/golden/int8_worked_example.json),
    through the row quantizer and through the paged write at slot 2;
  * round half away from zero on exact ties (the INT8 write fix) and the
    clamp to [-128, 127];
  * the dequantisation error bound |q s - x| <= s/2 (plus fp32 slack), the
    absmax element at +-127, the 1e-6 scale floor on a zero row;
  * agreement with an independent numpy transcription of the printed
    reference quantizer (torch.round: half to even) on random rows;
  * negative slots skipped, rows at the layout's offsets;
  * attention equal to a numpy brute force over numpy-decoded rows, with a
    window and a soft cap too; a single key returns its value row.
"""
import json
import os

import numpy as np
import pytest
import torch

from int4_quantized_paged_amd import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden", "int8_worked_example.json")


def _bf16_bits(x):
    return wl.bits16(torch.tensor(x, dtype=torch.bfloat16))


def test_worked_example_row(oracle_mod):
    g = json.load(open(GOLD))
    x = torch.tensor(g["key_as_printed"], dtype=torch.bfloat16).float().numpy()
    assert np.array_equal(x, np.array(g["key_bf16_values"], np.float32))
    codes, s = oracle_mod.quantize_row_int8(x)
    assert codes.tolist() == g["key_codes"] and s == g["scale"]
    codes, s = oracle_mod.quantize_row_int8(-x)
    assert codes.tolist() == g["value_codes"] and s == g["scale"]


def test_worked_example_paged_write(oracle_mod):
    g = json.load(open(GOLD))
    key = torch.tensor([g["key_as_printed"]], dtype=torch.bfloat16).view(1, 1, 8)
    cache = np.full(oracle_mod.cache_shape_int8(1, g["block_size"], 1, 8), 0xA5, np.uint8)
    oracle_mod.kv_write_int8(wl.bits16(key), wl.bits16(-key), "bf16", np.array([g["slot"]]), cache)
    off = g["slot"] % g["block_size"]
    for kv, name in ((0, "key_codes"), (1, "value_codes")):
        row = cache[0, kv, off, 0]
        assert row[:8].view(np.int8).tolist() == g[name]
        assert row[8:].view("<f4")[0] == np.float32(g["scale"])
    # every other row keeps the sentinel
    mask = np.ones(cache.shape[:4], bool)
    mask[0, :, off, 0] = False
    assert np.all(cache[mask] == 0xA5)


def test_ties_round_half_away_from_zero(oracle_mod):
    x = np.array([127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 0], np.float32)
    codes, s = oracle_mod.quantize_row_int8(x)
    assert s == 1.0
    assert codes.tolist() == [127, 3, -3, 1, -1, 2, -2, 0]


def test_absmax_maps_to_127_and_error_bound(oracle_mod):
    rng = np.random.default_rng(3)
    for d in (64, 128):
        for scale in (1e-3, 1.0, 300.0):
            for _ in range(50):
                x = (rng.standard_normal(d) * scale).astype(np.float32)
                codes, s = oracle_mod.quantize_row_int8(x)
                assert s == np.float32(max(np.float32(np.abs(x).max()) / np.float32(127), 1e-6))
                i = int(np.abs(x).argmax())
                assert abs(int(codes[i])) == 127 and np.sign(codes[i]) == np.sign(x[i])
                err = np.abs(codes.astype(np.float64) * s - x.astype(np.float64))
                assert err.max() <= s * (0.5 + 2.0 ** -20)


def test_zero_row_floor(oracle_mod):
    codes, s = oracle_mod.quantize_row_int8(np.zeros(64, np.float32))
    assert s == np.float32(1e-6) and not codes.any()


def test_agrees_with_printed_reference(oracle_mod):
    """numpy transcription of the page's reference: absmax / 127, clamp(min=1e-6),
    x * (1 / s), torch.round (half to even), clamp to [-128, 127]."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2000, 128)).astype(np.float32)
    s = np.maximum(np.abs(x).max(axis=1) / np.float32(127), np.float32(1e-6)).astype(np.float32)
    ref = np.clip(np.round(x * (np.float32(1) / s)[:, None]), -128, 127).astype(np.int64)
    got = np.stack([oracle_mod.quantize_row_int8(r)[0] for r in x]).astype(np.int64)
    assert np.abs(got - ref).max() <= 1
    assert (got == ref).mean() >= 0.999


def test_negative_slots_and_offsets(oracle_mod):
    w = wl.custom([(1, 40)], 8, 2, 64, seed=2, write_all=True)
    idx, slots = w.token_set("all")
    slots = slots.numpy().copy()
    slots[::3] = -1
    cache = np.full(oracle_mod.cache_shape_int8(w.num_blocks, 16, 2, 64), 0x5A, np.uint8)
    oracle_mod.kv_write_int8(wl.bits16(w.key[idx]), wl.bits16(w.value[idx]), "bf16", slots, cache)
    for t, sl in enumerate(slots):
        for kv, src in ((0, w.key), (1, w.value)):
            for h in range(2):
                row = cache[sl // 16, kv, sl % 16, h] if sl >= 0 else None
                if sl < 0:
                    continue
                codes, s = oracle_mod.quantize_row_int8(src[idx[t], h].float().numpy())
                assert np.array_equal(row[:64].view(np.int8), codes)
                assert row[64:].view("<f4")[0] == np.float32(s)
    written = np.zeros(cache.shape[:4], bool)
    for sl in slots[slots >= 0]:
        written[sl // 16, :, sl % 16, :] = True
    assert np.all(cache[~written] == 0x5A)


def _build(oracle_mod, w):
    cache = np.zeros(oracle_mod.cache_shape_int8(w.num_blocks, 16, w.num_kv_heads, w.head_size),
                     np.uint8)
    idx, slots = w.token_set("all")
    dt = "bf16" if w.dtype == torch.bfloat16 else "f16"
    oracle_mod.kv_write_int8(wl.bits16(w.key[idx]), wl.bits16(w.value[idx]), dt, slots.numpy(),
                             cache)
    return cache, dt


def _numpy_brute(w, cache, window=0, softcap=0.0):
    d = w.head_size
    G = w.num_q_heads // w.num_kv_heads
    q = w.query.float().numpy().astype(np.float64)
    out = np.zeros(q.shape)
    cu = w.cu_seqlens_q().tolist()

    def dec(blk, kv, off, h):
        row = cache[blk, kv, off, h]
        return row[:d].view(np.int8).astype(np.float64) * float(row[d:].view("<f4")[0])

    for b in range(w.num_seqs):
        L, ql = w.kv_lens[b], w.query_lens[b]
        for h in range(w.num_kv_heads):
            K = np.stack([dec(int(w.block_table[b, j // 16]), 0, j % 16, h) for j in range(L)])
            V = np.stack([dec(int(w.block_table[b, j // 16]), 1, j % 16, h) for j in range(L)])
            for i in range(ql):
                pos = L - ql + i
                lo = max(0, pos - window + 1) if window > 0 else 0
                for g in range(h * G, (h + 1) * G):
                    z = w.softmax_scale * (K[lo: pos + 1] @ q[cu[b] + i, g])
                    if softcap > 0:
                        z = softcap * np.tanh(z / softcap)
                    p = np.exp(z - z.max())
                    out[cu[b] + i, g] = (p / p.sum()) @ V[lo: pos + 1]
    return out


@pytest.mark.parametrize("window,softcap", [(0, 0.0), (20, 0.0), (0, 3.0)])
@pytest.mark.parametrize("d,hq,hkv", [(64, 4, 1), (128, 8, 2)])
def test_attention_matches_numpy_brute_force(oracle_mod, window, softcap, d, hq, hkv):
    w = wl.custom([(1, 17), (3, 33), (1, 1), (2, 48)], hq, hkv, d, seed=d + hq, write_all=True,
                  scale=2.0)
    cache, dt = _build(oracle_mod, w)
    got = oracle_mod.attention_plain_int8(wl.bits16(w.query), dt, cache, w.cu_seqlens_q().numpy(),
                                          w.seqused_k().numpy(), w.block_table.numpy(),
                                          w.softmax_scale, w.num_q_heads, window=window,
                                          softcap=softcap)
    np.testing.assert_allclose(got, _numpy_brute(w, cache, window, softcap), rtol=0, atol=1e-10)


def test_single_key_returns_value(oracle_mod):
    w = wl.custom([(1, 1), (1, 1)], 4, 2, 128, seed=9, write_all=True)
    cache, dt = _build(oracle_mod, w)
    out = oracle_mod.attention_plain_int8(wl.bits16(w.query), dt, cache, w.cu_seqlens_q().numpy(),
                                          w.seqused_k().numpy(), w.block_table.numpy(),
                                          w.softmax_scale, w.num_q_heads)
    for b in range(2):
        blk = int(w.block_table[b, 0])
        for g in range(4):
            v = oracle_mod.decode_row_int8(cache[blk, 1, 0, g // 2], 128)
            np.testing.assert_allclose(out[b, g], v, rtol=0, atol=1e-12)

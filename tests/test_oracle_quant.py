"""Pins of the oracle's per-row quantizer and cache write.

Checks: hand-worked examples (tests/golden/worked_examples.json), the
dequantization error bound, code endpoints, agreement with an independent
numpy transcription of the printed reference quantizer, the paged row address
against a numpy view of the cache shape, and negative-slot skipping.
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _f32(bits):
    return float(np.array([bits], np.uint32).view(np.float32)[0])


def _decode_row_codes(row, d):
    codes = np.empty(d, np.int64)
    codes[0::2] = row[: d // 2] & 0xF
    codes[1::2] = row[: d // 2] >> 4
    word = int(np.frombuffer(row[d // 2: d // 2 + 4].tobytes(), "<u4")[0])
    return codes, word & 0xF, _f32(word & 0xFFFFFFF0), word


def test_worked_example_d4(oracle_mod):
    ex = [e for e in json.load(open(GOLD))["examples"] if e["name"] == "d4_ramp"][0]
    y = oracle_mod.rht_forward_f32(np.array(ex["x"], np.float32), np.array(ex["signs"], np.float32))
    assert y.tolist() == ex["y"]
    b, w = oracle_mod.quantize_row(y)
    assert w == int(ex["scale_word"], 16)
    row = np.concatenate([b, np.frombuffer(np.uint32(w).tobytes(), np.uint8)])
    assert row.tobytes().hex() == ex["row_bytes_hex"]
    codes, zp, _, _ = _decode_row_codes(row, 4)
    assert codes.tolist() == ex["codes"] and zp == 4


def test_worked_example_zero_row(oracle_mod):
    ex = [e for e in json.load(open(GOLD))["examples"] if e["name"] == "d64_zero"][0]
    b, w = oracle_mod.quantize_row(np.zeros(64, np.float32))
    row = np.concatenate([b, np.frombuffer(np.uint32(w).tobytes(), np.uint8)])
    assert w == int(ex["scale_word"], 16)
    assert row.tobytes().hex() == ex["row_bytes_hex"]


def _rows(seed, n, d):
    r = np.random.default_rng(seed)
    ys = [r.standard_normal((n, d)) * 11.3,
          r.standard_normal((n, d)) * np.exp(r.uniform(-8, 8, (n, 1))),
          r.uniform(-1, 3, (n, d)),
          np.round(r.standard_normal((n, d)) * 4) / 2]  # many exact ties
    return np.concatenate(ys).astype(np.float32)


@pytest.mark.parametrize("d", [64, 128])
def test_error_bound_and_endpoints(oracle_mod, d):
    ys = _rows(d, 300, d)
    checked = 0
    for y in ys:
        b, w = oracle_mod.quantize_row(y)
        row = np.concatenate([b, np.frombuffer(np.uint32(w).tobytes(), np.uint8)])
        codes, zp, st, _ = _decode_row_codes(row, d)
        mn, mx = float(y.min()), float(y.max())
        if not (mn <= 0.0 <= mx):
            continue
        s = np.float32((np.float32(mx) - np.float32(mn)) / np.float32(15.0))
        if s <= np.float32(1e-6):
            continue
        checked += 1
        err = np.abs((codes - zp) * np.float64(st) - y.astype(np.float64))
        assert err.max() <= st * (0.5 + 2.0 ** -14)
        assert codes[int(np.argmin(y))] == 0
        assert codes[int(np.argmax(y))] in (14, 15)
        assert 0 <= zp <= 15
    assert checked > 600


def test_agrees_with_printed_reference_formula(oracle_mod):
    """Independent numpy transcription of the reference quantizer printed in
    the test file (section 6): untruncated scale, true division, round half to
    even.  The oracle quantizes with the truncated scale and a reciprocal, so
    codes may differ by one at near-ties only."""
    ys = _rows(99, 400, 128)
    total = diff = 0
    for ri, y in enumerate(ys):
        continuous = ri < 3 * 400  # the last family is built of exact ties
        mn, mx = np.float32(y.min()), np.float32(y.max())
        s = np.maximum(np.float32((mx - mn) / np.float32(15.0)), np.float32(1e-6))
        zp = np.clip(np.round(np.float32(-mn / s)), 0, 15)
        ref = np.clip(np.round((y / s).astype(np.float32) + np.float32(zp)), 0, 15).astype(np.int64)
        b, w = oracle_mod.quantize_row(y)
        codes = np.empty(128, np.int64)
        codes[0::2] = b & 0xF
        codes[1::2] = b >> 4
        assert w & 0xF == int(zp) or abs((w & 0xF) - int(zp)) <= 1
        if continuous:
            total += 128
            diff += int((codes != ref).sum())
        assert np.abs(codes - ref).max() <= 1
    assert diff / total <= 1e-3


def _sentinel_cache(nb, bs, hkv, d, fill=0xA5):
    return np.full((nb, 2, bs, hkv, d // 2 + 4), fill, np.uint8)


def test_row_address_matches_cache_view(oracle_mod):
    # d4 worked example written as the V of head 1 at slot 5 (block 1, offset 1)
    ex = [e for e in json.load(open(GOLD))["examples"] if e["name"] == "d4_ramp"][0]
    nb, bs, hkv, d = 3, 4, 2, 4
    x = np.array(ex["x"], np.float16)
    key = np.zeros((1, hkv, d), np.float16)
    val = np.zeros((1, hkv, d), np.float16)
    val[0, 1] = x
    cache = _sentinel_cache(nb, bs, hkv, d)
    oracle_mod.kv_write(key.view(np.uint16), val.view(np.uint16), "f16",
                        np.array([5], np.int64), cache, np.array(ex["signs"], np.float32))
    assert cache[1, 1, 1, 1].tobytes().hex() == ex["row_bytes_hex"]
    zero_row = oracle_mod.quantize_row(np.zeros(4, np.float32))
    assert cache[1, 0, 1, 0, :2].tolist() == zero_row[0].tolist()
    # flat byte offset (((blk*2 + kv)*B + off)*Hkv + h)*R, written out by hand
    flat = cache.reshape(-1)
    o = (((1 * 2 + 1) * 4 + 1) * 2 + 1) * 6
    assert flat[o:o + 6].tobytes().hex() == ex["row_bytes_hex"]
    # exactly one token's rows (2 kinds x 2 heads) changed
    changed = (cache != 0xA5).any(-1).sum()
    assert changed == 4


def test_bf16_and_f16_inputs_decode_exactly(oracle_mod):
    # small integers are exact in both 16-bit formats: same bytes either way
    d = 64
    r = np.random.default_rng(0)
    xi = r.integers(-8, 9, size=(3, 2, d)).astype(np.float32)
    s = (r.integers(0, 2, d) * 2 - 1).astype(np.float32)
    c1 = _sentinel_cache(1, 16, 2, d)
    c2 = _sentinel_cache(1, 16, 2, d)
    f16 = xi.astype(np.float16).view(np.uint16)
    bf = (xi.view(np.uint32) >> 16).astype(np.uint16)
    slots = np.array([0, 3, 7], np.int64)
    oracle_mod.kv_write(f16, f16, "f16", slots, c1, s)
    oracle_mod.kv_write(bf, bf, "bf16", slots, c2, s)
    assert np.array_equal(c1, c2)


def test_negative_slots_leave_cache_untouched(oracle_mod):
    nb, bs, hkv, d = 2, 16, 2, 64
    r = np.random.default_rng(1)
    k = r.standard_normal((4, hkv, d)).astype(np.float16).view(np.uint16)
    v = r.standard_normal((4, hkv, d)).astype(np.float16).view(np.uint16)
    s = np.ones(d, np.float32)
    cache = _sentinel_cache(nb, bs, hkv, d)
    before = cache.copy()
    oracle_mod.kv_write(k, v, "f16", np.array([0, -1, 1, -1], np.int64), cache, s)
    assert not np.array_equal(cache[0, 0, 0], before[0, 0, 0])
    assert not np.array_equal(cache[0, 1, 1], before[0, 1, 1])
    assert np.array_equal(cache[0, :, 2:], before[0, :, 2:])
    assert np.array_equal(cache[1], before[1])
    # written rows are exactly tokens 0 and 2
    c2 = _sentinel_cache(nb, bs, hkv, d)
    oracle_mod.kv_write(k[[0, 2]], v[[0, 2]], "f16", np.array([0, 1], np.int64), c2, s)
    assert np.array_equal(cache, c2)


def test_decode_row_matches_numpy_dequant(oracle_mod):
    """oracle.decode_row against an independent numpy dequant: codes from the
    nibbles, zp and scale from the word, inverse rotation as a matrix product."""
    from tests.test_oracle_rht import sylvester
    d = 128
    r = np.random.default_rng(4)
    s = (r.integers(0, 2, d) * 2 - 1).astype(np.float32)
    x = r.standard_normal((1, 1, d)).astype(np.float16)
    cache = _sentinel_cache(1, 16, 1, d)
    oracle_mod.kv_write(x.view(np.uint16), x.view(np.uint16), "f16", np.array([3], np.int64),
                        cache, s)
    row = cache[0, 0, 3, 0]
    codes, zp, st, _ = _decode_row_codes(row, d)
    yhat = (codes - zp) * st
    ref = s.astype(np.float64) * (sylvester(d) @ yhat) / d
    got = oracle_mod.decode_row(row, d, s)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    # and the dequantized row is close to the input (4-bit quantization error)
    err = np.abs(got - x[0, 0].astype(np.float64))
    assert err.max() < 0.6 * st and np.sqrt((err ** 2).mean()) < 0.5 * st

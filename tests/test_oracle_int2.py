"""Pins of the oracle's INT2 Lloyd-Max mode (rows of d/4 code bytes and an fp32
scale over the INT4 mode's rotation; readings R2-layout, R2-rot, R2-lm,
R2-scale, R2-deq):

  * the 4-level Lloyd-Max quantizer of N(0, 1) against the published table
    (Max, "Quantizing for minimum distortion", IRE Trans. Inform. Theory 6,
    1960, Table I, N = 4: levels 0.4528 and 1.510, threshold 0.9816, mean
    squared error 0.1175) and against its optimality conditions evaluated by
    numerical integration (scipy.integrate.quad, not the oracle's closed forms);
  * the scale within one ulp of the exact RMS of the row, the 1e-6 floor;
  * codes equal to the nearest level by brute force (argmin), ties upward,
    and the bit layout (element 4j + k in bits 2k, 2k+1 of byte j);
  * the distortion of Gaussian rows near the table's 0.1175;
  * decoding equal to an independent numpy decoding through scipy's Hadamard
    matrix; negative slots skipped; attention equal to a numpy brute force.
"""
import math

import numpy as np
import pytest
import torch
from scipy import integrate
from scipy.linalg import hadamard
from scipy.stats import norm

from int4_quantized_paged_amd import workloads as wl


def test_lloyd_max_matches_the_published_table(oracle_mod):
    a, b, t = oracle_mod.lloyd_max4()
    assert abs(a - 0.4528) < 5e-5
    assert abs(b - 1.510) < 5e-4
    assert abs(t - 0.9816) < 5e-5


def _mse(a, b, t):
    f = lambda lo, hi, c: integrate.quad(lambda x: (x - c) ** 2 * norm.pdf(x), lo, hi,
                                         epsabs=1e-13, epsrel=1e-13)[0]
    return 2 * (f(0, t, a) + f(t, np.inf, b))


def test_lloyd_max_optimality_conditions(oracle_mod):
    a, b, t = oracle_mod.lloyd_max4()
    m = lambda lo, hi: (integrate.quad(lambda x: x * norm.pdf(x), lo, hi, epsabs=1e-14)[0] /
                        (norm.cdf(hi) - norm.cdf(lo)))
    assert abs(a - m(0, t)) < 1e-9  # level = conditional mean of its cell
    assert abs(b - m(t, np.inf)) < 1e-9
    assert abs(t - (a + b) / 2) < 1e-12  # threshold = midpoint
    mse = _mse(a, b, t)
    assert abs(mse - 0.1175) < 1e-4
    for da, db in ((1e-3, 0), (-1e-3, 0), (0, 1e-3), (0, -1e-3)):  # a local minimum
        aa, bb = a + da, b + db
        assert _mse(aa, bb, (aa + bb) / 2) > mse


def _unpack(row_bytes, d):
    return np.array([(int(row_bytes[i // 4]) >> (2 * (i % 4))) & 3 for i in range(d)])


@pytest.mark.parametrize("d", [64, 128])
def test_quantizer_nearest_level_and_scale(oracle_mod, d):
    a, b, t = oracle_mod.lloyd_max4()
    levels = np.array([-b, -a, a, b])
    rng = np.random.default_rng(d)
    checked = 0
    for r in range(200):
        y = (rng.standard_normal(d) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        if r % 7 == 0:
            y[rng.integers(d)] *= 40.0  # an outlier
        by, s = oracle_mod.quantize_row_int2(y)
        rms = math.sqrt(float(np.mean(y.astype(np.float64) ** 2)))
        assert abs(s - rms) <= 2 * np.spacing(np.float32(rms))
        codes = _unpack(by, d)
        v = y.astype(np.float64) / s
        near = np.abs(np.abs(v)[:, None] - np.array([0.0, t])[None, :]).min(axis=1) < 1e-5
        want = np.argmin(np.abs(v[:, None] - levels[None, :]), axis=1)
        assert np.array_equal(codes[~near], want[~near])
        checked += int((~near).sum())
    assert checked > 0.99 * 200 * d


def test_quantizer_exact_cases_and_layout(oracle_mod):
    a, b, t = oracle_mod.lloyd_max4()
    # |y| = 3 everywhere: s = 3, v = +-1 >= t: codes 3 and 0
    y = np.array([3.0, -3.0] * 32, np.float32)
    by, s = oracle_mod.quantize_row_int2(y)
    assert s == 3.0
    assert by.tolist() == [0b00110011] * 16  # elements 0, 2 -> 3; 1, 3 -> 0
    # zero row: the 1e-6 floor; v = 0 sits on the middle threshold -> code 2
    by, s = oracle_mod.quantize_row_int2(np.zeros(64, np.float32))
    assert s == np.float32(1e-6) and by.tolist() == [0b10101010] * 16
    # one value per code at known positions (s fixed by the rest of the row)
    y = np.zeros(64, np.float32)
    y[:4] = [-1.5, -0.5, 0.5, 1.5]
    y[4:] = 1.0
    by, s = oracle_mod.quantize_row_int2(y)
    inv = np.float32(1) / np.float32(s)
    v = (y[:4] * inv).astype(np.float64)
    want = [int(np.argmin(np.abs(x - np.array([-b, -a, a, b])))) for x in v]
    assert want == [0, 1, 2, 3]
    assert by[0] == 0 | (1 << 2) | (2 << 4) | (3 << 6)


def test_gaussian_rows_reach_the_table_distortion(oracle_mod):
    a, b, _ = oracle_mod.lloyd_max4()
    levels = np.array([-b, -a, a, b])
    rng = np.random.default_rng(7)
    err = []
    for _ in range(400):
        y = rng.standard_normal(128).astype(np.float32)
        by, s = oracle_mod.quantize_row_int2(y)
        yh = s * levels[_unpack(by, 128)]
        err.append(np.mean((yh - y) ** 2) / np.mean(y.astype(np.float64) ** 2))
    assert abs(np.mean(err) - 0.1175) < 0.006


def _dec_numpy(row, d, signs, levels):
    codes = _unpack(row[: d // 4], d)
    s = float(np.frombuffer(row[d // 4:].tobytes(), "<f4")[0])
    return signs.astype(np.float64) * (hadamard(d).astype(np.float64) @ (s * levels[codes])) / d


@pytest.mark.parametrize("d", [64, 128])
def test_write_and_decode_against_numpy(oracle_mod, d):
    a, b, _ = oracle_mod.lloyd_max4()
    levels = np.array([-b, -a, a, b])
    g = torch.Generator().manual_seed(d)
    T, hkv, nb = 9, 2, 2
    key = torch.randn((T, hkv, d), generator=g).to(torch.bfloat16)
    value = (3 * torch.randn((T, hkv, d), generator=g)).to(torch.bfloat16)
    signs = wl.rht_signs(d).numpy()
    slots = np.array([0, 5, -1, 17, 31, 2, -1, 16, 30], np.int64)
    cache = np.full(oracle_mod.cache_shape_int2(nb, 16, hkv, d), 0xA5, np.uint8)
    oracle_mod.kv_write_int2(wl.bits16(key), wl.bits16(value), "bf16", slots, cache, signs)
    written = set()
    for t_, sl in enumerate(slots):
        if sl < 0:
            continue
        for kv, src in ((0, key), (1, value)):
            for h in range(hkv):
                row = cache[sl // 16, kv, sl % 16, h]
                written.add((sl // 16, kv, sl % 16, h))
                x = src[t_, h].float().numpy()
                # fp64 Hadamard product, rounded once: equal to the fp32
                # butterflies whenever no partial sum needs more than 24 bits
                # (true for these bf16 rows)
                y = (hadamard(d).astype(np.float64) @ (x * signs).astype(np.float64)).astype(np.float32)
                by, s = oracle_mod.quantize_row_int2(y)
                assert np.array_equal(row[: d // 4], by)
                got = oracle_mod.decode_row_int2(row, d, signs)
                assert np.allclose(got, _dec_numpy(row, d, signs, levels), rtol=0, atol=1e-12)
                # the round trip keeps the row's direction (INT2: cosine > 0.8)
                cos = got @ x / (np.linalg.norm(got) * np.linalg.norm(x))
                assert cos > 0.8
    for idx in np.ndindex(nb, 2, 16, hkv):
        if idx not in written:
            assert (cache[idx] == 0xA5).all()


def test_attention_against_numpy_brute_force(oracle_mod):
    a, b, _ = oracle_mod.lloyd_max4()
    levels = np.array([-b, -a, a, b])
    w = wl.custom([(1, 37), (4, 21), (3, 3)], 8, 2, 64, seed=3, write_all=True)
    d, B = 64, 16
    signs = w.signs.numpy()
    cache = np.zeros(oracle_mod.cache_shape_int2(w.num_blocks, B, 2, d), np.uint8)
    idx, slots = w.token_set("all")
    oracle_mod.kv_write_int2(wl.bits16(w.key[idx]), wl.bits16(w.value[idx]), "bf16",
                             slots.numpy(), cache, signs)
    q = w.query.float().numpy().astype(np.float64)
    cu = w.cu_seqlens_q().tolist()
    for window, cap in ((0, 0.0), (5, 0.0), (0, 2.0)):
        got = oracle_mod.attention_plain_int2(wl.bits16(w.query), "bf16", cache,
                                              w.cu_seqlens_q().numpy(), w.seqused_k().numpy(),
                                              w.block_table.numpy(), w.softmax_scale, signs, 8,
                                              window=window, softcap=cap)
        want = np.zeros_like(got)
        for bq in range(w.num_seqs):
            L, ql = w.kv_lens[bq], w.query_lens[bq]
            for h in range(2):
                rows = lambda kv: np.stack([_dec_numpy(cache[int(w.block_table[bq, j // B]), kv,
                                                             j % B, h], d, signs, levels)
                                            for j in range(L)])
                K, V = rows(0), rows(1)
                for i in range(ql):
                    pos = L - ql + i
                    lo = max(0, pos - window + 1) if window > 0 else 0
                    for g in range(4 * h, 4 * h + 4):
                        z = w.softmax_scale * (K[lo: pos + 1] @ q[cu[bq] + i, g])
                        if cap > 0:
                            z = cap * np.tanh(z / cap)
                        p = np.exp(z - z.max())
                        want[cu[bq] + i, g] = (p / p.sum()) @ V[lo: pos + 1]
        assert np.allclose(got, want, rtol=0, atol=1e-10), (window, cap)

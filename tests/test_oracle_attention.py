"""Pins of the oracle's two attention formulations.

* attention_plain (textbook softmax attention over the decoded cache) against
  an independent numpy brute force that decodes rows with numpy views and a
  matrix-form inverse Hadamard transform;
* attention_method (rotated-domain split-dot score with the sum(Q)*zp term,
  per-block online softmax, split-K segments merged by a segment reduction,
  inverse rotation) against attention_plain, to 1e-9;
* closed-form special cases: a single key, identical keys, causal masking,
  segment-count invariance, prefill row vs decode at the same position.
"""
import numpy as np
import pytest
import torch

from int4_quantized_paged_amd import workloads as wl
from tests.test_oracle_rht import sylvester


def _build_cache(oracle_mod, w):
    cache = np.zeros(oracle_mod.cache_shape(w.num_blocks, w.block_size, w.num_kv_heads,
                                            w.head_size), np.uint8)
    idx, slots = w.token_set("all")
    oracle_mod.kv_write(wl.bits16(w.key[idx]), wl.bits16(w.value[idx]),
                        "bf16" if w.dtype == torch.bfloat16 else "f16", slots.numpy(), cache,
                        w.signs.numpy())
    return cache


def _dt(w):
    return "bf16" if w.dtype == torch.bfloat16 else "f16"


def _run(oracle_mod, w, cache, method=False, ns=1):
    args = (wl.bits16(w.query), _dt(w), cache, w.cu_seqlens_q().numpy(), w.seqused_k().numpy(),
            w.block_table.numpy(), w.softmax_scale, w.signs.numpy(), w.num_q_heads)
    if method:
        return oracle_mod.attention_method(*args, num_segments=ns)
    return oracle_mod.attention_plain(*args)


def _numpy_brute(w, cache, softcap=0.0):
    d, B = w.head_size, w.block_size
    H = sylvester(d).astype(np.float64)
    sg = w.signs.numpy().astype(np.float64)
    G = w.num_q_heads // w.num_kv_heads
    q = w.query.float().numpy().astype(np.float64)
    out = np.zeros(q.shape)
    cu = w.cu_seqlens_q().tolist()

    def dec(blk, kv, off, h):
        row = cache[blk, kv, off, h]
        codes = np.empty(d)
        codes[0::2] = row[: d // 2] & 0xF
        codes[1::2] = row[: d // 2] >> 4
        word = int(np.frombuffer(row[d // 2:].tobytes(), "<u4")[0])
        st = float(np.array([word & 0xFFFFFFF0], np.uint32).view(np.float32)[0])
        return sg * (H @ ((codes - (word & 0xF)) * st)) / d

    for b in range(w.num_seqs):
        L, ql = w.kv_lens[b], w.query_lens[b]
        for h in range(w.num_kv_heads):
            K = np.stack([dec(int(w.block_table[b, j // B]), 0, j % B, h) for j in range(L)])
            V = np.stack([dec(int(w.block_table[b, j // B]), 1, j % B, h) for j in range(L)])
            for i in range(ql):
                pos = L - ql + i
                for g in range(h * G, (h + 1) * G):
                    z = w.softmax_scale * (K[: pos + 1] @ q[cu[b] + i, g])
                    if softcap > 0:
                        z = softcap * np.tanh(z / softcap)
                    p = np.exp(z - z.max())
                    out[cu[b] + i, g] = (p / p.sum()) @ V[: pos + 1]
    return out


CASES = [
    dict(lens=[(1, 42)], hq=1, hkv=1, d=64, dtype=torch.float16),
    dict(lens=[(1, 17), (3, 33), (1, 1)], hq=4, hkv=1, d=64, dtype=torch.bfloat16),
    dict(lens=[(5, 48), (2, 16)], hq=8, hkv=1, d=128, dtype=torch.bfloat16),
    dict(lens=[(1, 30), (4, 21)], hq=8, hkv=2, d=128, dtype=torch.bfloat16),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_plain_matches_numpy_brute_force(oracle_mod, case):
    c = CASES[case]
    w = wl.custom(c["lens"], c["hq"], c["hkv"], c["d"], dtype=c["dtype"], seed=case, write_all=True)
    cache = _build_cache(oracle_mod, w)
    got = _run(oracle_mod, w, cache)
    ref = _numpy_brute(w, cache)
    assert np.allclose(got, ref, rtol=0, atol=1e-10)


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("ns", [1, 2, 3, 5])
def test_method_matches_plain(oracle_mod, case, ns):
    c = CASES[case]
    w = wl.custom(c["lens"], c["hq"], c["hkv"], c["d"], dtype=c["dtype"], seed=10 + case,
                  write_all=True)
    cache = _build_cache(oracle_mod, w)
    plain = _run(oracle_mod, w, cache)
    meth = _run(oracle_mod, w, cache, method=True, ns=ns)
    assert np.abs(meth - plain).max() <= 1e-9


def test_single_key_returns_its_value(oracle_mod):
    w = wl.custom([(1, 1)], 4, 1, 128, seed=3, write_all=True)
    cache = _build_cache(oracle_mod, w)
    out = _run(oracle_mod, w, cache)
    blk = int(w.block_table[0, 0])
    v0 = oracle_mod.decode_row(cache[blk, 1, 0, 0], 128, w.signs.numpy())
    for g in range(4):
        assert np.allclose(out[0, g], v0, rtol=0, atol=1e-12)


def test_identical_keys_give_mean_of_values(oracle_mod):
    w = wl.custom([(1, 40)], 2, 1, 64, seed=4, write_all=True)
    w.key[:] = w.key[0:1]  # every key identical -> uniform softmax weights
    cache = _build_cache(oracle_mod, w)
    out = _run(oracle_mod, w, cache)
    s = w.signs.numpy()
    V = np.stack([oracle_mod.decode_row(cache[int(w.block_table[0, j // 16]), 1, j % 16, 0], 64, s)
                  for j in range(40)])
    assert np.allclose(out[0, 0], V.mean(0), rtol=0, atol=1e-12)
    assert np.allclose(out[0, 1], V.mean(0), rtol=0, atol=1e-12)


def test_keys_after_position_are_ignored(oracle_mod):
    # prefill of 6 queries over 30 keys: perturbing key 29 (visible only to the
    # last query) changes only the last query's output
    w = wl.custom([(6, 30)], 4, 2, 64, seed=5, write_all=True)
    cache = _build_cache(oracle_mod, w)
    out1 = _run(oracle_mod, w, cache)
    w.key[29] = -w.key[29] * 3
    w.value[29] = w.value[29] * 2 + 1
    cache2 = _build_cache(oracle_mod, w)
    out2 = _run(oracle_mod, w, cache2)
    assert np.array_equal(out1[:5], out2[:5])
    assert np.abs(out1[5] - out2[5]).max() > 1e-3


def test_prefill_row_equals_decode_at_same_position(oracle_mod):
    w = wl.custom([(7, 37)], 8, 2, 128, seed=6, write_all=True)
    cache = _build_cache(oracle_mod, w)
    out = _run(oracle_mod, w, cache)
    for i in range(7):
        dq = wl.Workload(w.name, w.dtype, w.num_q_heads, w.num_kv_heads, w.head_size,
                         w.num_blocks, [37 - 6 + i], [1], [1], w.block_table, w.key, w.value,
                         w.query[i:i + 1], w.signs)
        o = _run(oracle_mod, dq, cache)
        assert np.abs(o[0] - out[i]).max() <= 1e-12


def test_gqa_head_mapping(oracle_mod):
    # with G = 4, query heads 0..3 read KV head 0 and 4..7 read KV head 1:
    # giving KV head 1 the same K/V as KV head 0 makes the two groups agree
    w = wl.custom([(1, 20)], 8, 2, 64, seed=8, write_all=True)
    w.key[:, 1] = w.key[:, 0]
    w.value[:, 1] = w.value[:, 0]
    w.query[:, 4:] = w.query[:, :4]
    cache = _build_cache(oracle_mod, w)
    out = _run(oracle_mod, w, cache)
    assert np.array_equal(out[0, :4], out[0, 4:])
    w.value[:, 1] = -w.value[:, 1]
    cache = _build_cache(oracle_mod, w)
    out2 = _run(oracle_mod, w, cache)
    assert np.array_equal(out2[0, :4], out[0, :4])
    assert not np.allclose(out2[0, 4:], out[0, 4:])


def test_segments_invariance_on_long_sequence(oracle_mod):
    w = wl.custom([(1, 700), (1, 129)], 4, 1, 64, seed=9, write_all=True)
    cache = _build_cache(oracle_mod, w)
    ref = _run(oracle_mod, w, cache, method=True, ns=1)
    for ns in [2, 7, 16, 64]:  # 64 > blocks of the short sequence: empty segments
        got = _run(oracle_mod, w, cache, method=True, ns=ns)
        assert np.abs(got - ref).max() <= 1e-12

"""Pins of the oracle's logit soft-capping (R-cap: each scaled score z becomes
c * tanh(z / c) before the softmax; the pull request's packed read path
shares the common kernel's softcap helper):

  * a cap far above every logit, or c <= 0, is no capping;
  * a cap far below every logit flattens the softmax: the output is the mean
    of the visible decoded value rows;
  * a single visible key returns its decoded value row whatever the cap;
  * the capped plain formulation equals an independent numpy brute force
    (numpy row decoding, matrix-form inverse Hadamard transform, np.tanh);
  * the method formulation (rotated-domain split dot, online softmax, split-K
    segments) agrees with the plain one under the cap.
"""
import numpy as np
import pytest

from int4_quantized_paged_amd import workloads as wl
from tests.test_oracle_attention import _build_cache, _dt, _numpy_brute


def _attn(oracle_mod, w, cache, softcap, method=False, ns=1, window=0):
    args = (wl.bits16(w.query), _dt(w), cache, w.cu_seqlens_q().numpy(), w.seqused_k().numpy(),
            w.block_table.numpy(), w.softmax_scale, w.signs.numpy(), w.num_q_heads)
    if method:
        return oracle_mod.attention_method(*args, num_segments=ns, window=window,
                                           softcap=softcap)
    return oracle_mod.attention_plain(*args, window=window, softcap=softcap)


def _mixed(scale=1.0, d=64):
    # inputs scaled so that the logits reach tens: the cap matters
    return wl.custom([(1, 70), (3, 40), (1, 17), (5, 100)], 8, 2, d, seed=41, scale=scale)


@pytest.mark.parametrize("cap", [0.0, -1.0, 1e12])
def test_huge_or_no_cap_is_no_cap(oracle_mod, cap):
    w = _mixed(scale=3.0)
    cache = _build_cache(oracle_mod, w)
    ref = _attn(oracle_mod, w, cache, 0.0)
    np.testing.assert_allclose(_attn(oracle_mod, w, cache, cap), ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(_attn(oracle_mod, w, cache, cap, method=True, ns=3),
                               _attn(oracle_mod, w, cache, 0.0, method=True, ns=3),
                               rtol=0, atol=1e-12)


def test_tiny_cap_gives_mean_of_values(oracle_mod):
    w = _mixed(scale=3.0)
    cache = _build_cache(oracle_mod, w)
    out = _attn(oracle_mod, w, cache, 1e-9)
    G = w.num_q_heads // w.num_kv_heads
    cu = w.cu_seqlens_q().tolist()
    sg = w.signs.numpy()
    for b in range(w.num_seqs):
        L, ql = w.kv_lens[b], w.query_lens[b]
        for h in range(w.num_kv_heads):
            V = np.stack([oracle_mod.decode_row(cache[int(w.block_table[b, j // 16]), 1, j % 16, h],
                                                w.head_size, sg) for j in range(L)])
            for i in range(ql):
                pos = L - ql + i
                for g in range(h * G, (h + 1) * G):
                    np.testing.assert_allclose(out[cu[b] + i, g], V[: pos + 1].mean(axis=0),
                                               rtol=0, atol=1e-7)


def test_single_key_ignores_cap(oracle_mod):
    w = wl.custom([(1, 1), (1, 1)], 4, 2, 128, seed=5, scale=10.0)
    cache = _build_cache(oracle_mod, w)
    for cap in (0.5, 3.0, 50.0):
        np.testing.assert_allclose(_attn(oracle_mod, w, cache, cap), _attn(oracle_mod, w, cache, 0),
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("cap", [1.0, 5.0, 30.0])
@pytest.mark.parametrize("d", [64, 128])
def test_capped_plain_matches_numpy_brute_force(oracle_mod, cap, d):
    w = _mixed(scale=3.0, d=d)
    cache = _build_cache(oracle_mod, w)
    got = _attn(oracle_mod, w, cache, cap)
    ref = _numpy_brute(w, cache, softcap=cap)
    assert np.allclose(got, ref, rtol=0, atol=1e-10)
    # and the cap changes the result at these logits (the pin is not vacuous)
    assert np.abs(got - _attn(oracle_mod, w, cache, 0.0)).max() > 1e-3


@pytest.mark.parametrize("ns", [1, 2, 5])
@pytest.mark.parametrize("window", [0, 20])
def test_capped_method_matches_plain(oracle_mod, ns, window):
    w = _mixed(scale=3.0, d=128)
    cache = _build_cache(oracle_mod, w)
    plain = _attn(oracle_mod, w, cache, 4.0, window=window)
    meth = _attn(oracle_mod, w, cache, 4.0, method=True, ns=ns, window=window)
    np.testing.assert_allclose(meth, plain, rtol=0, atol=1e-9)

"""Pins of the oracle's sliding window (R-win: the query at position pos sees
keys [pos - W + 1, pos]; the pull request's read path shares the common
kernel's sliding-window masking helper):

  * a window at least as long as every sequence, or W <= 0, is no window;
  * W = 1 returns the decoded value row of the query's own position;
  * dropping whole blocks from the front of the block table (seqused_k cut
    to W) gives the same result as the window when L - W is a multiple of 16;
  * the method formulation (rotated-domain split dot, online softmax, split-K
    segments starting at the first visible block) agrees with the plain one.
"""
import numpy as np
import pytest
import torch

from int4_quantized_paged_amd import workloads as wl
from tests.test_oracle_attention import _build_cache, _dt


def _attn(oracle_mod, w, cache, window, method=False, ns=1, block_table=None, seqused=None):
    bt = w.block_table.numpy() if block_table is None else block_table
    su = w.seqused_k().numpy() if seqused is None else seqused
    args = (wl.bits16(w.query), _dt(w), cache, w.cu_seqlens_q().numpy(), su, bt,
            w.softmax_scale, w.signs.numpy(), w.num_q_heads)
    if method:
        return oracle_mod.attention_method(*args, num_segments=ns, window=window)
    return oracle_mod.attention_plain(*args, window=window)


def _mixed():
    return wl.custom([(1, 70), (3, 40), (1, 17), (5, 100)], 8, 2, 64, seed=31)


@pytest.mark.parametrize("window", [0, -3, 100, 1000])
def test_long_or_no_window_is_no_window(oracle_mod, window):
    w = _mixed()
    cache = _build_cache(oracle_mod, w)
    ref = _attn(oracle_mod, w, cache, 0)
    assert np.array_equal(_attn(oracle_mod, w, cache, window), ref)
    assert np.array_equal(_attn(oracle_mod, w, cache, window, method=True, ns=3),
                          _attn(oracle_mod, w, cache, 0, method=True, ns=3))


def test_window_one_returns_own_value(oracle_mod):
    w = _mixed()
    cache = _build_cache(oracle_mod, w)
    out = _attn(oracle_mod, w, cache, 1)
    G = w.num_q_heads // w.num_kv_heads
    cu = w.cu_seqlens_q().tolist()
    sg = w.signs.numpy()
    for b in range(w.num_seqs):
        L, ql = w.kv_lens[b], w.query_lens[b]
        for i in range(ql):
            pos = L - ql + i
            blk = int(w.block_table[b, pos // 16])
            for g in range(w.num_q_heads):
                v = oracle_mod.decode_row(cache[blk, 1, pos % 16, g // G], w.head_size, sg)
                np.testing.assert_allclose(out[cu[b] + i, g], v, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("L,W", [(80, 32), (80, 64), (208, 16), (200, 8 + 16 * 3)])
def test_window_equals_dropped_leading_blocks(oracle_mod, L, W):
    """Decode query at pos = L - 1; when L - W is a multiple of 16, the first
    (L - W) / 16 blocks can be cut from the block table instead."""
    if (L - W) % 16:
        pytest.skip("only block-aligned drops are expressible as a block table")
    w = wl.custom([(1, L)], 8, 2, 128, seed=L + W)
    cache = _build_cache(oracle_mod, w)
    win = _attn(oracle_mod, w, cache, W)
    drop = (L - W) // 16
    bt = np.ascontiguousarray(w.block_table.numpy()[:, drop:])
    cut = _attn(oracle_mod, w, cache, 0, block_table=bt, seqused=np.array([W], np.int32))
    assert np.array_equal(win, cut)


@pytest.mark.parametrize("window", [1, 5, 16, 17, 33, 64])
@pytest.mark.parametrize("ns", [1, 3, 8])
def test_method_matches_plain_with_window(oracle_mod, window, ns):
    w = _mixed()
    cache = _build_cache(oracle_mod, w)
    ref = _attn(oracle_mod, w, cache, window)
    got = _attn(oracle_mod, w, cache, window, method=True, ns=ns)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10)


def test_window_changes_the_result(oracle_mod):
    """A window shorter than the context must matter (guards against a
    window argument that is silently ignored)."""
    w = _mixed()
    cache = _build_cache(oracle_mod, w)
    assert not np.allclose(_attn(oracle_mod, w, cache, 8), _attn(oracle_mod, w, cache, 0))

"""GPU parity of sliding-window attention (the query at position pos sees
keys [pos - W + 1, pos]) against the oracle: decode (LDS-staged kernel at
several group sizes and head sizes, split-K segments starting at the first
visible block, the register path for 3 KV heads), prefill/mixed batches, and
the fused decode step; a window at least as long as every sequence gives the
same bits as no window."""
import pytest
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import (assert_attention_close, gpu_attention, gpu_cache, gpu_write, header,
                               oracle_attention, oracle_cache, to_dev)

pytestmark = pytest.mark.gpu

DECODE_LENS = [(1, 1), (1, 16), (1, 17), (1, 100), (1, 517), (1, 2000)]


@pytest.mark.parametrize("hq,hkv,d", [(64, 8, 128), (32, 8, 64), (16, 4, 128), (8, 2, 64),
                                      (6, 3, 128), (128, 8, 128)])
def test_decode_window(oracle_mod, hq, hkv, d):
    w = wl.custom(DECODE_LENS, hq, hkv, d, seed=hq + 7 * hkv + d, write_all=True)
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    ref_cache = oracle_cache(oracle_mod, w, "all")
    for window in (1, 16, 17, 100, 600):
        ref = oracle_attention(oracle_mod, w, ref_cache, window=window)
        for ns in (1, 4, 16):
            header(f"decode window {window} {hq}/{hkv} d{d} NS={ns}")
            out = gpu_attention(w, t, c, ns, window=window)
            torch.cuda.synchronize()
            assert_attention_close(out, ref, f"window {window} NS={ns}")


@pytest.mark.parametrize("G,d", [(4, 128), (8, 64), (1, 128)])
def test_prefill_window(oracle_mod, G, d):
    lens = [(40, 120), (9, 300), (1, 77), (33, 33), (100, 700)]
    w = wl.custom(lens, G * 2, 2, d, seed=G + d, write_all=True)
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    ref_cache = oracle_cache(oracle_mod, w, "all")
    for window in (1, 7, 32, 33, 200):
        header(f"prefill window {window} G={G} d{d}")
        out = gpu_attention(w, t, c, 1, window=window)
        torch.cuda.synchronize()
        assert_attention_close(out, oracle_attention(oracle_mod, w, ref_cache, window=window),
                               f"window {window}")


def test_long_window_is_no_window(oracle_mod):
    w = wl.custom([(1, 300), (1, 45), (7, 90)], 32, 8, 128, seed=3, write_all=True)
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    for ns in (1, 4):
        a = gpu_attention(w, t, c, ns)
        b = gpu_attention(w, t, c, ns, window=300)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    wd = wl.custom([(1, 300), (1, 45)], 32, 8, 128, seed=3, write_all=True)
    td = to_dev(wd)
    cd = gpu_cache(wd)
    gpu_write(wd, td, cd, "all")
    for ns in (1, 8):
        a = gpu_attention(wd, td, cd, ns)
        b = gpu_attention(wd, td, cd, ns, window=10 ** 6)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_decode_step_window(oracle_mod):
    """The fused step with a window: the new token's block is found from the
    first visible block on."""
    w = wl.custom([(1, 2000), (1, 300), (1, 17)], 64, 8, 128, seed=41)
    t = to_dev(w)
    prior_idx, prior_slots = w.token_set("prior")
    new_idx, new_slots = w.token_set("new")
    c = gpu_cache(w)
    ik.int4_kv_write(t["key"][prior_idx.cuda()], t["value"][prior_idx.cuda()], prior_slots.cuda(),
                     c, t["signs"])
    ref_cache = oracle_cache(oracle_mod, w, "all")
    for window, ns in ((100, 4), (500, 16), (33, 1)):
        header(f"decode step window {window} NS={ns}")
        cc = c.clone()
        segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size, device="cuda")
        out = ik.int4_decode_step(t["key"][new_idx.cuda()], t["value"][new_idx.cuda()],
                                  new_slots.cuda(), t["query"], cc, t["cu"], t["su"], 1,
                                  w.max_seqlen_k, t["block_table"], w.softmax_scale, t["signs"],
                                  num_segments=ns, segm_output=segs[0], segm_max=segs[1],
                                  segm_expsum=segs[2], sliding_window=window)
        torch.cuda.synchronize()
        assert torch.equal(cc.cpu(), torch.from_numpy(ref_cache))
        assert_attention_close(out, oracle_attention(oracle_mod, w, ref_cache, window=window),
                               f"step window {window}")

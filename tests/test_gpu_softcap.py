"""GPU parity of logit soft-capping (scores z become c * tanh(z / c) before
the softmax) against the oracle: decode (LDS-staged kernel at several group
and head sizes, split-K, the register path for 3 KV heads, with a sliding
window too), prefill/mixed batches and the fused decode step.  Inputs are
scaled by 3 so that the logits reach tens and every cap tested changes the
result (checked, so the cases are not vacuous)."""
import numpy as np
import pytest
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import (assert_attention_close, gpu_attention, gpu_cache, gpu_write, header,
                               oracle_attention, oracle_cache, to_dev)

pytestmark = pytest.mark.gpu

DECODE_LENS = [(1, 1), (1, 16), (1, 17), (1, 100), (1, 517), (1, 2000)]
CAPS = (1.0, 5.0, 30.0)


def _changes(ref, ref_uncapped):
    assert np.abs(ref - ref_uncapped).max() > 1e-2, "the cap does not change this case"


@pytest.mark.parametrize("hq,hkv,d", [(64, 8, 128), (32, 8, 64), (16, 4, 128), (6, 3, 128)])
def test_decode_softcap(oracle_mod, hq, hkv, d):
    w = wl.custom(DECODE_LENS, hq, hkv, d, seed=hq + 5 * hkv + d, write_all=True, scale=3.0)
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    ref_cache = oracle_cache(oracle_mod, w, "all")
    plain = oracle_attention(oracle_mod, w, ref_cache)
    for cap in CAPS:
        ref = oracle_attention(oracle_mod, w, ref_cache, softcap=cap)
        _changes(ref, plain)
        for ns in (1, 4):
            header(f"decode softcap {cap} {hq}/{hkv} d{d} NS={ns}")
            out = gpu_attention(w, t, c, ns, softcap=cap)
            torch.cuda.synchronize()
            assert_attention_close(out, ref, f"softcap {cap} NS={ns}")


def test_decode_softcap_with_window(oracle_mod):
    w = wl.custom(DECODE_LENS, 32, 8, 128, seed=77, write_all=True, scale=3.0)
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    ref_cache = oracle_cache(oracle_mod, w, "all")
    ref = oracle_attention(oracle_mod, w, ref_cache, window=100, softcap=5.0)
    for ns in (1, 16):
        header(f"decode softcap 5 window 100 NS={ns}")
        out = gpu_attention(w, t, c, ns, window=100, softcap=5.0)
        torch.cuda.synchronize()
        assert_attention_close(out, ref, f"softcap + window NS={ns}")


@pytest.mark.parametrize("G,d", [(4, 128), (8, 64), (1, 128)])
def test_prefill_softcap(oracle_mod, G, d):
    lens = [(40, 120), (9, 300), (1, 77), (33, 33), (100, 700)]
    w = wl.custom(lens, G * 2, 2, d, seed=G + 3 * d, write_all=True, scale=3.0)
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    ref_cache = oracle_cache(oracle_mod, w, "all")
    plain = oracle_attention(oracle_mod, w, ref_cache)
    for cap in CAPS:
        header(f"prefill softcap {cap} G={G} d{d}")
        ref = oracle_attention(oracle_mod, w, ref_cache, softcap=cap)
        _changes(ref, plain)
        out = gpu_attention(w, t, c, 1, softcap=cap)
        torch.cuda.synchronize()
        assert_attention_close(out, ref, f"softcap {cap}")


def test_decode_step_softcap(oracle_mod):
    """The fused step with a cap: the cache bytes and the output of the two
    calls, bit for bit, and the oracle's capped attention."""
    w = wl.custom([(1, 300), (1, 41), (1, 1500), (1, 17)], 64, 8, 128, seed=33, scale=3.0)
    t = to_dev(w)
    ca, cb = gpu_cache(w), gpu_cache(w)
    gpu_write(w, t, ca, "prior")
    gpu_write(w, t, cb, "prior")
    new_idx, new_slots = w.token_set("new")
    kn, vn = t["key"][new_idx.cuda()], t["value"][new_idx.cuda()]
    slots = new_slots.cuda()
    for ns in (1, 4):
        header(f"fused step softcap NS={ns}")
        ik.int4_kv_write(kn, vn, slots, ca, t["signs"])
        out_a = gpu_attention(w, t, ca, ns, softcap=5.0)
        segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size, device="cuda") \
            if ns > 1 else (None, None, None)
        out_b = ik.int4_decode_step(kn, vn, slots, t["query"], cb, t["cu"], t["su"], 1,
                                    w.max_seqlen_k, t["block_table"], w.softmax_scale, t["signs"],
                                    num_segments=ns, segm_output=segs[0], segm_max=segs[1],
                                    segm_expsum=segs[2], softcap=5.0)
        torch.cuda.synchronize()
        assert torch.equal(ca, cb)
        assert torch.equal(out_a, out_b)
    ref = oracle_attention(oracle_mod, w, oracle_cache(oracle_mod, w, "all"), softcap=5.0)
    assert_attention_close(out_b, ref, "fused step softcap")

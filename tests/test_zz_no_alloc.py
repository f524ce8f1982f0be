"""int4_paged_attention_noalloc (split-K partials in the library's fixed device
buffer, nothing allocated) against int4_paged_attention with caller-owned
segment buffers: bit for bit, on two calls in a row, the second one smaller,
and both against the oracle at |gpu - ref| <= 2e-3 + 1e-2 |ref|."""
import numpy as np
import pytest
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import (assert_attention_close, gpu_attention, gpu_cache, gpu_write, header,
                               oracle_attention, oracle_cache, to_dev)

pytestmark = pytest.mark.gpu


def _noalloc(w, t, cache, ns, out):
    return ik.int4_paged_attention_noalloc(t["query"], cache, t["cu"], t["su"], w.max_seqlen_q,
                                           w.max_seqlen_k, t["block_table"], w.softmax_scale,
                                           t["signs"], out, num_segments=ns)


def test_noalloc_matches_caller_buffers_two_calls(oracle_mod):
    cases = [
        (wl.custom([(1, 3000), (1, 1700), (1, 50), (1, 1), (1, 777)], 64, 8, 128, seed=41,
                   write_all=True), 16),
        (wl.custom([(1, 200), (1, 33)], 32, 8, 128, seed=42, write_all=True), 4),
    ]
    for i, (w, ns) in enumerate(cases):
        header(f"noalloc call {i}: {w.name} NS={ns}")
        t = to_dev(w)
        c = gpu_cache(w)
        gpu_write(w, t, c, "all")
        ref_out = gpu_attention(w, t, c, ns)  # caller-owned segment buffers
        out = torch.full_like(t["query"], float("nan"))
        _noalloc(w, t, c, ns, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"call {i}: differs from int4_paged_attention"
        ref = oracle_attention(oracle_mod, w, oracle_cache(oracle_mod, w, "all"))
        assert_attention_close(out, ref, f"noalloc call {i}")


def test_noalloc_one_segment_and_prefill(oracle_mod):
    """No partials are used with one segment or a prefill batch."""
    for w, ns in ((wl.custom([(1, 90), (1, 300)], 16, 4, 64, seed=43, write_all=True), 1),
                  (wl.custom([(20, 90), (7, 300)], 16, 4, 64, seed=44, write_all=True), 8)):
        header(f"noalloc {w.name} NS={ns}")
        t = to_dev(w)
        c = gpu_cache(w)
        gpu_write(w, t, c, "all")
        out = torch.empty_like(t["query"])
        _noalloc(w, t, c, ns, out)
        torch.cuda.synchronize()
        assert torch.equal(out, gpu_attention(w, t, c, ns))


def test_noalloc_rejects_partials_beyond_the_buffer():
    """4 x 64 query heads x 256 segments x d 128 need 33 MB of partials: the call
    is refused before anything is enqueued."""
    w = wl.custom([(1, 64)] * 4, 64, 8, 128, seed=45, write_all=True)
    t = to_dev(w)
    c = gpu_cache(w)
    out = torch.zeros_like(t["query"])
    with pytest.raises(ik.Int4KVError) as e:
        _noalloc(w, t, c, 256, out)
    assert e.value.status == 3  # INT4KV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out == 0)

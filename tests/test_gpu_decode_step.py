"""GPU parity of the fused decode step (int4_decode_step): the same cache
bytes and the same output, bit for bit, as int4_kv_write of the new tokens
followed by int4_paged_attention; and within the attention bound of the
oracle.  Covers the fused kernel (KV-head counts 2, 4, 8, 16), the
two-launch fallback (3 KV heads; query lengths > 1), new tokens at block
boundaries, split counts that put the last key in the first or a later
segment, skipped slots and sequences without a query."""
import pytest
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import (assert_attention_close, gpu_attention, gpu_cache, gpu_write, header,
                               oracle_attention, oracle_cache, to_dev)

pytestmark = pytest.mark.gpu

LENS = [(1, 1), (1, 16), (1, 17), (1, 300), (1, 513), (1, 2000)]


def _split(w, t, skip=()):
    """Every key but each sequence's last, written beforehand; and the last key
    of each sequence as the step's new token: key_new / value_new [S, Hkv, d]
    and slots [S], slot -1 (zeros) where the sequence has no key or is listed
    in ``skip``."""
    S, dev = w.num_seqs, t["key"].device
    off = w.token_offsets()
    pidx, pslots = [], []
    kn = torch.zeros((S, w.num_kv_heads, w.head_size), dtype=w.dtype, device=dev)
    vn = torch.zeros_like(kn)
    slots = torch.full((S,), -1, dtype=torch.int64)
    for b in range(S):
        L = w.kv_lens[b]
        if L < 1:
            continue
        if L > 1:
            pos = torch.arange(0, L - 1, dtype=torch.int64)
            pidx.append(pos + off[b])
            pslots.append(w.slots_of(b, pos))
        if b in skip:
            continue
        kn[b] = t["key"][off[b] + L - 1]
        vn[b] = t["value"][off[b] + L - 1]
        slots[b] = w.slots_of(b, torch.tensor([L - 1]))[0]
    base = gpu_cache(w)
    if pidx:
        idx = torch.cat(pidx).to(dev)
        ik.int4_kv_write(t["key"][idx], t["value"][idx], torch.cat(pslots).to(dev), base,
                         t["signs"])
    return base, kn, vn, slots.to(dev)


def _both(w, ns, skip=()):
    t = to_dev(w)
    base, kn, vn, slots = _split(w, t, skip)
    ca, cb = base.clone(), base.clone()
    ik.int4_kv_write(kn, vn, slots, ca, t["signs"])
    out_a = gpu_attention(w, t, ca, ns)
    segs = (None, None, None)
    if ns > 1 and w.max_seqlen_q == 1:
        segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size, device="cuda")
    out_b = ik.int4_decode_step(kn, vn, slots, t["query"], cb, t["cu"], t["su"], w.max_seqlen_q,
                                w.max_seqlen_k, t["block_table"], w.softmax_scale, t["signs"],
                                num_segments=ns, segm_output=segs[0], segm_max=segs[1],
                                segm_expsum=segs[2])
    torch.cuda.synchronize()
    assert torch.equal(ca, cb), "cache bytes differ from the separate write"
    assert torch.equal(out_a, out_b), "output differs from the separate calls"
    return out_b


@pytest.mark.parametrize("hq,hkv,d,dtype,ns_list", [
    (64, 8, 128, torch.bfloat16, [1, 4, 64]),
    (32, 8, 128, torch.float16, [1, 16]),
    (32, 8, 64, torch.bfloat16, [1, 16]),
    (16, 4, 128, torch.bfloat16, [1, 4]),
    (8, 2, 64, torch.bfloat16, [1, 3]),
    (32, 16, 128, torch.bfloat16, [1, 8]),
    (128, 8, 128, torch.bfloat16, [1, 8]),
    (6, 3, 128, torch.bfloat16, [1, 4]),
])
def test_decode_step_matches_two_calls(oracle_mod, hq, hkv, d, dtype, ns_list):
    w = wl.custom(LENS, hq, hkv, d, dtype=dtype, seed=hq + 3 * hkv + d)
    for ns in ns_list:
        header(f"decode step {hq}/{hkv} d{d} {dtype} NS={ns}")
        _both(w, ns)


def test_decode_step_against_oracle(oracle_mod):
    w = wl.custom(LENS, 64, 8, 128, seed=5)
    header("decode step vs oracle NS=16")
    out = _both(w, 16)
    ref = oracle_attention(oracle_mod, w, oracle_cache(oracle_mod, w, "all"))
    assert_attention_close(out, ref, "fused decode step")


def test_decode_step_skips_and_empty_queries(oracle_mod):
    """Sequence 1 has no query (its new token is still written), sequence 3's
    slot is -1 (nothing written: its last key keeps the fill bytes), sequence
    4 has no keys at all."""
    w = wl.custom([(1, 40), (0, 20), (1, 33), (1, 70), (1, 0), (1, 16)], 32, 8, 128, seed=9)
    for ns in (1, 4):
        header(f"decode step skips NS={ns}")
        _both(w, ns, skip=(3,))


def test_decode_step_prefill_batch_falls_back(oracle_mod):
    """max_seqlen_q > 1: the write, then the prefill path (two launches)."""
    w = wl.custom([(1, 50), (5, 90), (1, 17)], 32, 8, 128, seed=13)
    header("decode step with a prefill row")
    _both(w, 1)


def test_decode_step_serving_batch(oracle_mod):
    """100 sequences of 514-640 keys at the library's split count (2): the
    fused step against the two calls bit for bit, and 10 sampled sequences
    against the oracle."""
    w = wl.serving_standin()
    ns = ik.int4kv_decode_num_segments(w.num_seqs, w.num_kv_heads, w.max_seqlen_k)
    assert ns == 2
    header(f"decode step serving batch NS={ns}")
    out = _both(w, ns)
    g = torch.Generator().manual_seed(12)
    picks = torch.randperm(w.num_seqs, generator=g)[:10].tolist()
    from tests.gpu_helpers import sub_workload
    ws = sub_workload(w, picks)
    ref = oracle_attention(oracle_mod, ws, oracle_cache(oracle_mod, ws, "all"))
    assert_attention_close(out[picks], ref, "serving batch, sampled sequences")


def test_decode_step_plan_matches_plain_call(oracle_mod):
    """DecodeStepPlan (arguments checked once) launches the same step: the
    same cache bytes and output bits as int4_decode_step, on repeated calls,
    after the buffers' contents change, and on a non-default stream."""
    w = wl.custom(LENS, 64, 8, 128, seed=9)
    t = to_dev(w)
    base, kn, vn, slots = _split(w, t)
    ns = 8
    segs = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size, device="cuda")
    ca, cb = base.clone(), base.clone()
    out_a, out_b = torch.empty_like(t["query"]), torch.empty_like(t["query"])
    plan = ik.DecodeStepPlan(kn, vn, slots, t["query"], cb, t["cu"], t["su"], w.max_seqlen_q,
                             w.max_seqlen_k, t["block_table"], w.softmax_scale, t["signs"],
                             out=out_b, num_segments=ns, segm_output=segs[0], segm_max=segs[1],
                             segm_expsum=segs[2])
    segs_a = ik.segment_buffers(w.num_seqs, w.num_q_heads, ns, w.head_size, device="cuda")

    def plain():
        ik.int4_decode_step(kn, vn, slots, t["query"], ca, t["cu"], t["su"], w.max_seqlen_q,
                            w.max_seqlen_k, t["block_table"], w.softmax_scale, t["signs"],
                            out=out_a, num_segments=ns, segm_output=segs_a[0],
                            segm_max=segs_a[1], segm_expsum=segs_a[2])
    for rnd in range(3):
        header(f"decode step plan, round {rnd}")
        if rnd == 1:  # new contents in the same buffers
            t["query"].mul_(-0.5)
            kn.mul_(2.0)
            vn.add_(0.25)
        if rnd == 2:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                plain()
                assert plan() is out_b
            torch.cuda.current_stream().wait_stream(s)
        else:
            plain()
            assert plan() is out_b
        torch.cuda.synchronize()
        assert torch.equal(ca, cb), "cache bytes differ from the plain call"
        assert torch.equal(out_a, out_b), "output differs from the plain call"

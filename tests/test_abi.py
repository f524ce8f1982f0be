"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function that include/int4kv.h declares,
size caches by the closed form, and reject invalid host arguments before
anything is enqueued (these calls never reach the GPU).
"""
import ctypes
import os
import re

import pytest

import int4_quantized_paged_amd as ik

HDR = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "int4kv.h")


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(int[248][a-z_0-9]*)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ik.load_library()
    names = declared_functions()
    assert {"int4_kv_write", "int4_paged_attention", "int4kv_cache_bytes",
            "int4kv_status_string", "int4kv_last_error", "int8_kv_write",
            "int8kv_cache_bytes", "int8_paged_attention", "int8kv_decode_num_segments",
            "int2kv_cache_bytes", "int2_kv_write"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    raw = ctypes.CDLL(ik.library_path())
    for n in names:
        assert ctypes.cast(getattr(raw, n), ctypes.c_void_p).value


@pytest.mark.parametrize("nb,bs,h,d", [(3, 16, 1, 64), (16384, 16, 8, 128), (1, 16, 8, 64)])
def test_cache_bytes_closed_form(nb, bs, h, d):
    assert ik.int4kv_cache_bytes(nb, bs, h, d) == nb * 2 * bs * h * (d // 2 + 4)


def test_cache_bytes_rejects_bad_dims():
    assert ik.int4kv_cache_bytes(0, 16, 1, 64) == -1
    assert ik.int4kv_cache_bytes(1, 16, 1, 63) == -1


def test_memory_ratio_vs_int8_and_bf16():
    # packed row d/2 + 4 bytes vs d + 4 (int8 per-token-head) and 2d (bf16)
    for d, r8 in [(128, 0.515), (64, 0.529)]:
        assert ik.int8kv_cache_bytes(1, 16, 1, d) == 2 * 16 * (d + 4)
        r = ik.int4kv_cache_bytes(1, 16, 1, d) / ik.int8kv_cache_bytes(1, 16, 1, d)
        assert abs(r - r8) < 1e-3
    assert abs(ik.int4kv_cache_bytes(1, 16, 1, 128) / (2 * 16 * 256) - 0.2656) < 1e-3


def test_status_strings():
    for code, name in [(0, "INT4KV_OK"), (1, "INT4KV_ERR_INVALID_ARG"), (2, "INT4KV_ERR_UNSUPPORTED"),
                       (3, "INT4KV_ERR_WORKSPACE"), (4, "INT4KV_ERR_LAUNCH")]:
        assert ik.int4kv_status_string(code) == name


FAKE = 0x10000  # 16-byte aligned non-null address; never dereferenced on these paths


def _write(**kw):
    a = dict(key=FAKE, ks=1024, value=FAKE, vs=1024, dtype=1, slots=FAKE, T=4, cache=FAKE, nb=4,
             bs=16, hkv=8, d=128, signs=FAKE, stream=None)
    a.update(kw)
    lib = ik.load_library()
    return lib.int4_kv_write(a["key"], a["ks"], a["value"], a["vs"], a["dtype"], a["slots"], a["T"],
                             a["cache"], a["nb"], a["bs"], a["hkv"], a["d"], a["signs"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(cache=None), 1), (dict(signs=None), 1), (dict(d=96), 2), (dict(d=256), 2),
    (dict(bs=32), 2), (dict(dtype=7), 1), (dict(T=-1), 1), (dict(key=None), 1),
    (dict(ks=1000), 1), (dict(vs=512), 1), (dict(key=FAKE + 2), 1), (dict(nb=0), 1),
])
def test_write_rejects_invalid_host_arguments(kw, status):
    assert _write(**kw) == status
    assert ik.int4kv_last_error() != ""


def test_write_zero_tokens_is_a_no_op():
    assert _write(T=0) == 0
    assert ik.int4kv_last_error() == ""


def _attn(**kw):
    a = dict(q=FAKE, qs=4096, out=FAKE, dtype=1, cache=FAKE, nb=64, bs=16, hkv=8, d=128, hq=32,
             cu=FAKE, su=FAKE, S=4, mq=1, mk=1024, bt=FAKE, bts=64, scale=0.088, win=0,
             cap=0.0, signs=FAKE, ns=1, so=None, sm=None, ss=None, stream=None)
    a.update(kw)
    lib = ik.load_library()
    return lib.int4_paged_attention(a["q"], a["qs"], a["out"], a["dtype"], a["cache"], a["nb"],
                                    a["bs"], a["hkv"], a["d"], a["hq"], a["cu"], a["su"], a["S"],
                                    a["mq"], a["mk"], a["bt"], a["bts"], a["scale"], a["win"],
                                    a["cap"], a["signs"], a["ns"], a["so"], a["sm"], a["ss"],
                                    a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(hq=30), 1), (dict(hq=24, hkv=8), 2), (dict(hq=256, hkv=8, qs=32768), 2),
    (dict(d=80), 2), (dict(bs=8), 2), (dict(ns=0), 1), (dict(ns=16), 3), (dict(bts=10), 1),
    (dict(qs=100), 1), (dict(out=None), 1), (dict(scale=float("inf")), 1), (dict(S=-1), 1),
    (dict(cache=FAKE + 4), 1), (dict(cap=float("nan")), 1), (dict(cap=float("inf")), 1),
    (dict(cap=1e-45), 1),
])
def test_attention_rejects_invalid_host_arguments(kw, status):
    assert _attn(**kw) == status
    assert ik.int4kv_last_error() != ""


def test_attention_empty_batch_is_a_no_op():
    assert _attn(S=0) == 0
    assert _attn(mq=0) == 0


def _step(**kw):
    a = dict(kn=FAKE, ks=1024, vn=FAKE, vs=1024, slots=FAKE, q=FAKE, qs=4096, out=FAKE, dtype=1,
             cache=FAKE, nb=64, bs=16, hkv=8, d=128, hq=32, cu=FAKE, su=FAKE, S=4, mq=1, mk=1024,
             bt=FAKE, bts=64, scale=0.088, win=0, cap=0.0, signs=FAKE, ns=1, so=None, sm=None,
             ss=None, stream=None)
    a.update(kw)
    lib = ik.load_library()
    return lib.int4_decode_step(a["kn"], a["ks"], a["vn"], a["vs"], a["slots"], a["q"], a["qs"],
                                a["out"], a["dtype"], a["cache"], a["nb"], a["bs"], a["hkv"],
                                a["d"], a["hq"], a["cu"], a["su"], a["S"], a["mq"], a["mk"],
                                a["bt"], a["bts"], a["scale"], a["win"], a["cap"], a["signs"], a["ns"],
                                a["so"], a["sm"], a["ss"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), 1), (dict(slots=None), 1), (dict(ks=100), 1), (dict(vn=FAKE + 2), 1),
    (dict(hq=30), 1), (dict(d=80), 2), (dict(ns=16), 3), (dict(cache=None), 1),
    (dict(dtype=5), 1), (dict(bts=10), 1), (dict(S=-1), 1),
])
def test_decode_step_rejects_invalid_host_arguments(kw, status):
    """The fused step validates both halves' arguments before enqueuing."""
    assert _step(**kw) == status
    assert ik.int4kv_last_error() != ""


def test_decode_step_empty_batch_is_a_no_op():
    assert _step(S=0) == 0


@pytest.mark.parametrize("S,hkv,L,ns", [
    (4, 8, 131072, 64),  # long-context decode: one workgroup per CU
    (64, 8, 4096, 4),    # Llama-3-8B-shaped decode: 256 workgroups
    (100, 8, 640, 2),    # serving stand-in: 3 segments would need a second round of 44
    (1, 8, 40, 1),       # shorter than two minimum segments
    (1, 8, 100, 1),      # 4 tiles: a split saves less than the reduction costs
    (8, 8, 1024, 16),    # GQA decode: capped by the minimum segment
    (32, 3, 5000, 8),    # register-path head count (one head per workgroup)
    (2, 16, 65536, 64),  # two workgroups per segment index
    (1, 1, 10 ** 7, 256),
])
def test_decode_num_segments_heuristic(S, hkv, L, ns):
    """The count with the fewest rounds of workgroups times (start + tiles per
    segment), plus the reduction for a split; none shorter than 2 tiles of 32
    keys, at most 256.  The benchmark shapes get the split counts that
    measured fastest (64, 4, 16 and 2)."""
    assert ik.int4kv_decode_num_segments(S, hkv, L) == ns


def test_decode_num_segments_fills_one_round_when_it_pays():
    """A split never makes a partial second round of workgroups for a batch
    whose sequences are short (the start and the reduction outweigh the
    shorter segments), and grows with the context once one round is full."""
    for S in (40, 64, 100, 128, 200):
        ns = ik.int4kv_decode_num_segments(S, 8, 640)
        assert ns * S <= 256 or ns == 1, (S, ns)
    grow = [ik.int4kv_decode_num_segments(4, 8, L) for L in (2048, 8192, 32768, 131072)]
    assert grow == sorted(grow) and grow[-1] == 64


def test_decode_num_segments_degenerate_inputs():
    for args in ((0, 8, 100), (4, 0, 100), (4, 8, 0), (-1, 8, 100)):
        assert ik.int4kv_decode_num_segments(*args) == 1


def _w8(**kw):
    a = dict(k=FAKE, ks=1024, v=FAKE, vs=1024, dtype=1, slots=FAKE, T=4, cache=FAKE, nb=64, bs=16,
             hkv=8, d=128, stream=None)
    a.update(kw)
    return ik.load_library().int8_kv_write(a["k"], a["ks"], a["v"], a["vs"], a["dtype"],
                                           a["slots"], a["T"], a["cache"], a["nb"], a["bs"],
                                           a["hkv"], a["d"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), 1), (dict(slots=None), 1), (dict(cache=None), 1), (dict(ks=100), 1),
    (dict(d=96), 2), (dict(bs=32), 2), (dict(dtype=7), 1), (dict(T=-1), 1),
    (dict(cache=FAKE + 8), 1), (dict(nb=0), 1),
])
def test_int8_write_rejects_invalid_host_arguments(kw, status):
    assert _w8(**kw) == status
    assert ik.int4kv_last_error() != ""


def test_int8_write_empty_is_a_no_op():
    assert _w8(T=0) == 0


def _a8(**kw):
    a = dict(q=FAKE, qs=4096, out=FAKE, dtype=1, cache=FAKE, nb=64, bs=16, hkv=8, d=128, hq=32,
             cu=FAKE, su=FAKE, S=4, mq=1, mk=1024, bt=FAKE, bts=64, scale=0.088, win=0, cap=0.0,
             ns=1, so=None, sm=None, ss=None, stream=None)
    a.update(kw)
    return ik.load_library().int8_paged_attention(
        a["q"], a["qs"], a["out"], a["dtype"], a["cache"], a["nb"], a["bs"], a["hkv"], a["d"],
        a["hq"], a["cu"], a["su"], a["S"], a["mq"], a["mk"], a["bt"], a["bts"], a["scale"],
        a["win"], a["cap"], a["ns"], a["so"], a["sm"], a["ss"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(hkv=3, hq=6), 2), (dict(mq=7, hq=24), 2), (dict(hkv=6, hq=12), 2), (dict(d=96), 2),
    (dict(bs=8), 2), (dict(hq=30), 1), (dict(ns=16), 3), (dict(cache=None), 1),
    (dict(cap=float("nan")), 1), (dict(bts=10), 1),
])
def test_int8_attention_rejects_invalid_host_arguments(kw, status):
    assert _a8(**kw) == status
    assert ik.int4kv_last_error() != ""


def test_int8_attention_empty_batch_is_a_no_op():
    assert _a8(S=0) == 0
    assert _a8(mq=0) == 0


@pytest.mark.parametrize("S,hkv,L,ns", [
    (64, 8, 4096, 2),    # Llama-3-8B-shaped: 4-head workgroups, 128 per segment index
    (4, 8, 131072, 32),
    (8, 8, 1024, 16),
    (1, 2, 100, 1),
])
def test_int8_decode_num_segments(S, hkv, L, ns):
    assert ik.int8kv_decode_num_segments(S, hkv, L) == ns


def _w2(**kw):
    a = dict(k=FAKE, ks=1024, v=FAKE, vs=1024, dtype=1, slots=FAKE, T=4, cache=FAKE, nb=64, bs=16,
             hkv=8, d=128, signs=FAKE, stream=None)
    a.update(kw)
    return ik.load_library().int2_kv_write(a["k"], a["ks"], a["v"], a["vs"], a["dtype"],
                                           a["slots"], a["T"], a["cache"], a["nb"], a["bs"],
                                           a["hkv"], a["d"], a["signs"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), 1), (dict(slots=None), 1), (dict(cache=None), 1), (dict(signs=None), 1),
    (dict(ks=100), 1), (dict(d=96), 2), (dict(bs=32), 2), (dict(dtype=7), 1), (dict(T=-1), 1),
    (dict(cache=FAKE + 8), 1), (dict(nb=0), 1),
])
def test_int2_write_rejects_invalid_host_arguments(kw, status):
    assert _w2(**kw) == status
    assert ik.int4kv_last_error() != ""


def test_int2_write_empty_is_a_no_op_and_cache_bytes():
    assert _w2(T=0) == 0
    assert ik.int2kv_cache_bytes(3, 16, 2, 128) == 3 * 2 * 16 * 2 * 36
    assert ik.int2kv_cache_bytes(1, 16, 1, 66) == -1


def _a2(**kw):
    a = dict(q=FAKE, qs=4096, out=FAKE, dtype=1, cache=FAKE, nb=64, bs=16, hkv=8, d=128, hq=32,
             cu=FAKE, su=FAKE, S=4, mq=1, mk=1024, bt=FAKE, bts=64, scale=0.088, win=0, cap=0.0,
             signs=FAKE, ns=1, so=None, sm=None, ss=None, stream=None)
    a.update(kw)
    return ik.load_library().int2_paged_attention(
        a["q"], a["qs"], a["out"], a["dtype"], a["cache"], a["nb"], a["bs"], a["hkv"], a["d"],
        a["hq"], a["cu"], a["su"], a["S"], a["mq"], a["mk"], a["bt"], a["bts"], a["scale"],
        a["win"], a["cap"], a["signs"], a["ns"], a["so"], a["sm"], a["ss"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(mq=7, hq=24), 2), (dict(hkv=3, hq=6), 2), (dict(hkv=12, hq=24), 2), (dict(d=96), 2),
    (dict(bs=8), 2), (dict(hq=30), 1), (dict(ns=16), 3), (dict(cache=None), 1),
    (dict(signs=None), 1), (dict(cap=float("nan")), 1), (dict(bts=10), 1),
])
def test_int2_attention_rejects_invalid_host_arguments(kw, status):
    assert _a2(**kw) == status
    assert ik.int4kv_last_error() != ""


def test_int2_attention_empty_batch_is_a_no_op():
    assert _a2(S=0) == 0
    assert _a2(mq=0) == 0


@pytest.mark.parametrize("args", [
    (FAKE, 32, FAKE, 0), (FAKE, 24, FAKE, 16), (FAKE, 16, FAKE, 8), (FAKE + 4, 16, FAKE, 16),
    (None, 16, FAKE, 16), (FAKE, 16, None, 16), (FAKE, -16, FAKE, 16),
])
def test_stream_rw_rejects_invalid_host_arguments(args):
    src, nr, dst, nw = args
    assert ik.load_library().int4kv_stream_rw(src, nr, dst, nw, None) == 1
    assert ik.int4kv_last_error() != ""


def test_stream_rw_empty_is_a_no_op():
    assert ik.load_library().int4kv_stream_rw(None, 0, None, 0, None) == 0


@pytest.mark.parametrize("args", [
    (FAKE, 17408, FAKE, 64, 0),          # no workgroups
    (FAKE, 17408, FAKE, -2, 1),          # negative count
    (FAKE, 1000, FAKE, 64, 4),           # block size not a multiple of 1024
    (FAKE, 0, FAKE, 64, 4),              # empty blocks
    (FAKE, 21504, FAKE, 64, 4),          # blocks past the ring's stage size
    (FAKE, 17408, FAKE, 66, 4),          # not whole tiles per workgroup
    (FAKE + 4, 17408, FAKE, 64, 4),      # misaligned cache
    (None, 17408, FAKE, 64, 4),          # null cache
    (FAKE, 17408, None, 64, 4),          # null ids
])
def test_stream_blocks_rejects_invalid_host_arguments(args):
    cache, bb, ids, n, wg = args
    assert ik.load_library().int4kv_stream_blocks(cache, bb, ids, n, wg, None) == 1
    assert ik.int4kv_last_error() != ""


def test_stream_blocks_empty_is_a_no_op():
    assert ik.load_library().int4kv_stream_blocks(None, 17408, None, 0, 4, None) == 0


def _plan_inputs(S=4, hkv=8, d=128, hq=32, nblk=8):
    import torch
    bf = torch.bfloat16
    return dict(key_new=torch.zeros(S, hkv, d, dtype=bf), value_new=torch.zeros(S, hkv, d, dtype=bf),
                slot_mapping=torch.zeros(S, dtype=torch.int64), q=torch.zeros(S, hq, d, dtype=bf),
                kv_cache=torch.zeros(S * nblk, 2, 16, hkv, d // 2 + 4, dtype=torch.uint8),
                cu_seqlens_q=torch.arange(S + 1, dtype=torch.int32),
                seqused_k=torch.full((S,), 100, dtype=torch.int32), max_seqlen_q=1,
                max_seqlen_k=100, block_table=torch.zeros(S, nblk, dtype=torch.int32),
                softmax_scale=0.088, rht_signs=torch.ones(d))


def test_decode_step_plan_converts_arguments_once():
    """DecodeStepPlan checks and converts its arguments at construction (host
    only: nothing is launched here): the C argument tuple has one value per
    declared argument but the stream, and ``out`` is allocated like q."""
    kw = _plan_inputs()
    plan = ik.DecodeStepPlan(**kw)
    lib = ik.load_library()
    assert len(plan._args) == len(lib.int4_decode_step.argtypes) - 1
    assert plan.out.shape == kw["q"].shape and plan.out.dtype == kw["q"].dtype
    assert plan._args[0].value == kw["key_new"].data_ptr()


@pytest.mark.parametrize("bad", [
    dict(slot_mapping="int32"), dict(key_new="3 tokens"), dict(block_table="int64"),
    dict(kv_cache="float"),
])
def test_decode_step_plan_rejects_what_the_plain_call_rejects(bad):
    import torch
    kw = _plan_inputs()
    (k, v), = bad.items()
    if k == "slot_mapping":
        kw[k] = kw[k].to(torch.int32)
    elif k == "key_new":
        kw[k] = kw[k][:3]
    elif k == "block_table":
        kw[k] = kw[k].to(torch.int64)
    else:
        kw[k] = kw[k].float()
    with pytest.raises(ValueError):
        ik.DecodeStepPlan(**kw)
    with pytest.raises(ValueError):
        ik.int4_decode_step(**kw)

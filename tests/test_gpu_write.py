"""GPU parity of the cache write: packed bytes and scale words must equal the
oracle's bit for bit, over the whole cache buffer (sentinel bytes included)."""
import random

import numpy as np
import pytest
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import SENTINEL, dt_name, gpu_cache, gpu_write, header, oracle_cache, to_dev

pytestmark = pytest.mark.gpu


def _write_both(oracle_mod, key, value, slots, nb, hkv, d, signs, key_dev=None, value_dev=None):
    dev = "cuda"
    c = torch.full(ik.cache_shape(nb, hkv, d), SENTINEL, dtype=torch.uint8, device=dev)
    ik.int4_kv_write(key.to(dev) if key_dev is None else key_dev,
                     value.to(dev) if value_dev is None else value_dev,
                     slots.to(dev), c, signs.to(dev))
    ref = np.full(oracle_mod.cache_shape(nb, 16, hkv, d), SENTINEL, np.uint8)
    oracle_mod.kv_write(wl.bits16(key), wl.bits16(value), "bf16" if key.dtype == torch.bfloat16
                        else "f16", slots.numpy(), ref, signs.numpy())
    torch.cuda.synchronize()
    return c.cpu().numpy(), ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hkv", [1, 4, 8])
@pytest.mark.parametrize("T", [1, 7, 42])
def test_write_page_grid_bit_exact(oracle_mod, T, hkv, d, dtype):
    header(f"write grid T={T} hkv={hkv} d={d} {dtype}")
    random.seed(0)
    g = torch.Generator().manual_seed(T * 100 + hkv * 10 + d)
    nb = (T + 15) // 16 + 4
    slots = torch.tensor(random.sample(range(nb * 16), T), dtype=torch.int64)
    key = torch.randn((T, hkv, d), generator=g).to(dtype)
    value = torch.randn((T, hkv, d), generator=g).to(dtype)
    got, ref = _write_both(oracle_mod, key, value, slots, nb, hkv, d, wl.rht_signs(d))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [4000, 4100])
def test_write_both_lane_layouts(oracle_mod, T, d):
    """8 KV heads: 4000 tokens (64000 rows) take the 16-elements-per-lane
    layout, 4100 tokens (65600 rows) the 32-elements-per-lane one; both bit
    for bit over the whole cache."""
    header(f"write lane layouts T={T} d={d}")
    random.seed(T + d)
    g = torch.Generator().manual_seed(T + d)
    nb = (T + 15) // 16 + 8
    slots = torch.tensor(random.sample(range(nb * 16), T), dtype=torch.int64)
    key = torch.randn((T, 8, d), generator=g).to(torch.bfloat16)
    value = (3.0 * torch.randn((T, 8, d), generator=g)).to(torch.bfloat16)
    got, ref = _write_both(oracle_mod, key, value, slots, nb, 8, d, wl.rht_signs(d))
    assert np.array_equal(got, ref)


def test_write_negative_slots(oracle_mod):
    header("write negative slots")
    g = torch.Generator().manual_seed(5)
    key = torch.randn((4, 2, 64), generator=g).to(torch.bfloat16)
    value = torch.randn((4, 2, 64), generator=g).to(torch.bfloat16)
    slots = torch.tensor([0, -1, 1, -1], dtype=torch.int64)
    got, ref = _write_both(oracle_mod, key, value, slots, 2, 2, 64, wl.rht_signs(64))
    assert np.array_equal(got, ref)
    assert (got[0, :, 2:] == SENTINEL).all() and (got[1] == SENTINEL).all()
    assert not (got[0, 0, 0] == SENTINEL).all()


@pytest.mark.parametrize("d", [64, 128])
def test_write_degenerate_rows(oracle_mod, d):
    """Zero rows (scale floor), constants, one-hot rows (rotated row constant
    up to sign), all-positive rotated rows (zp clamp), huge and tiny
    magnitudes, exact ties, fp16 subnormals."""
    header(f"write degenerate rows d={d}")
    rows = [torch.zeros(d), torch.full((d,), 3.0), torch.full((d,), -0.5),
            torch.nn.functional.one_hot(torch.tensor(0), d).float() * 7,
            torch.nn.functional.one_hot(torch.tensor(5), d).float() * -2,
            torch.arange(d).float() / 8, torch.randn(d) * 1e4, torch.randn(d) * 1e-5,
            torch.round(torch.randn(d) * 4) / 2, torch.full((d,), 6e-8)]
    x = torch.stack(rows)[:, None, :]
    for dtype in (torch.float16, torch.bfloat16):
        xx = x.to(dtype)
        T = xx.shape[0]
        slots = torch.arange(T, dtype=torch.int64) * 3
        got, ref = _write_both(oracle_mod, xx, -xx, slots, (3 * T) // 16 + 1, 1, d, wl.rht_signs(d))
        assert np.array_equal(got, ref), dtype


@pytest.mark.parametrize("d", [64, 128])
def test_write_degenerate_rows_bulk_layout(oracle_mod, d):
    """The degenerate rows above (plus exact half-integer grids) repeated over
    4100 tokens x 8 heads, so that they take the bulk lane layout."""
    header(f"write degenerate rows, bulk layout d={d}")
    g = torch.Generator().manual_seed(d)
    base = [torch.zeros(d), torch.full((d,), 3.0), torch.full((d,), -0.5),
            torch.nn.functional.one_hot(torch.tensor(0), d).float() * 7,
            torch.arange(d).float() / 8, torch.randn(d, generator=g) * 1e4,
            torch.randn(d, generator=g) * 1e-5, torch.round(torch.randn(d, generator=g) * 4) / 2,
            torch.full((d,), 6e-8), torch.round(torch.randn(d, generator=g) * 8) / 4]
    T, hkv = 4100, 8
    idx = torch.randint(0, len(base), (T, hkv), generator=g)
    rows = torch.stack(base)[idx] * torch.where(torch.rand(T, hkv, 1, generator=g) < 0.5, -1.0, 1.0)
    for dtype in (torch.float16, torch.bfloat16):
        xx = rows.to(dtype)
        nb = (T + 15) // 16 + 2
        slots = torch.randperm(nb * 16, generator=g)[:T].to(torch.int64)
        got, ref = _write_both(oracle_mod, xx, xx.flip(-1).contiguous(), slots, nb, hkv, d,
                               wl.rht_signs(d))
        assert np.array_equal(got, ref), dtype


def test_write_strided_token_layout(oracle_mod):
    """key/value as slices of a fused qkv tensor (token stride > heads * d)."""
    header("write strided qkv")
    g = torch.Generator().manual_seed(11)
    T, hq, hkv, d = 37, 32, 8, 128
    qkv = torch.randn((T, hq + 2 * hkv, d), generator=g).to(torch.bfloat16)
    qkv_d = qkv.cuda()
    key, value = qkv[:, hq:hq + hkv], qkv[:, hq + hkv:]
    key_d, value_d = qkv_d[:, hq:hq + hkv], qkv_d[:, hq + hkv:]
    slots = torch.randperm(64 * 16, generator=g)[:T].to(torch.int64)
    got, ref = _write_both(oracle_mod, key.contiguous(), value.contiguous(), slots, 64, hkv, d,
                           wl.rht_signs(d), key_dev=key_d, value_dev=value_d)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("make", [wl.tiny, wl.gqa_decode])
def test_write_small_workloads_whole_cache(oracle_mod, make):
    w = make()
    header(f"write workload {w.name}")
    t = to_dev(w)
    c = gpu_cache(w)
    gpu_write(w, t, c, "all")
    ref = oracle_cache(oracle_mod, w, "all")
    assert np.array_equal(c.cpu().numpy(), ref)


def test_write_llama3_bulk_fill_sampled(oracle_mod):
    """Full-size bulk fill (64 x 4096 tokens, 8 KV heads, d 128) in the launch
    configuration the benchmark times; 3000 sampled tokens checked against the
    oracle bit for bit, and every row of the cache written."""
    header("write Llama-3-8B-shaped bulk fill (sampled)")
    w = wl.llama3_8b_decode(device="cuda")
    idx, slots = w.token_set("all")
    c = gpu_cache(w)
    ik.int4_kv_write(w.key, w.value, slots.cuda(), c, w.signs.cuda())
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(1)
    pick = torch.randperm(idx.numel(), generator=g)[:3000]
    ref = np.full(oracle_mod.cache_shape(w.num_blocks, 16, 8, 128), SENTINEL, np.uint8)
    oracle_mod.kv_write(wl.bits16(w.key[pick.cuda()]), wl.bits16(w.value[pick.cuda()]), "bf16",
                        slots[pick].numpy(), ref, w.signs.numpy())
    s = slots[pick]
    blk, off = (s // 16).numpy(), (s % 16).numpy()
    got = c.cpu().numpy()
    assert np.array_equal(got[blk, :, off], ref[blk, :, off])
    # every (block, kv, offset, head) row was written: its scale word is a valid scale
    words = got[..., 64:68].copy().view("<u4")[..., 0]
    assert ((words & 0x7F800000) != 0x7F800000).all() and (words != 0xA5A5A5A5).all()


@pytest.mark.parametrize("mode", ["int4", "int8", "int2"])
def test_write_skips_slots_past_the_cache(oracle_mod, mode):
    """Slots at or beyond num_blocks * 16 are skipped like negative ones.  The
    cache handed to the library is the first NB blocks of a larger buffer, so
    a store that ignored the bound would land in the guard blocks behind it
    (inside this test's own allocation) and show there."""
    header(f"{mode} write: slots past the cache end are skipped")
    nb, guard, hkv, d, T = 6, 3, 4, 128, 40
    g = torch.Generator().manual_seed(91)
    key = torch.randn((T, hkv, d), generator=g).to(torch.bfloat16)
    value = torch.randn((T, hkv, d), generator=g).to(torch.bfloat16)
    random.seed(91)
    slots = torch.tensor(random.sample(range(nb * 16), T), dtype=torch.int64)
    slots[::4] = nb * 16 + torch.arange(0, T, 4) % (guard * 16)  # inside the guard blocks
    slots[1] = -1
    kept = slots.clone()
    kept[kept >= nb * 16] = -1
    shape = {"int4": ik.cache_shape, "int8": ik.cache_shape_int8,
             "int2": ik.cache_shape_int2}[mode](nb + guard, hkv, d)
    big = torch.full(shape, SENTINEL, dtype=torch.uint8, device="cuda")
    cache = big[:nb]
    signs = wl.rht_signs(d)
    if mode == "int4":
        ik.int4_kv_write(key.cuda(), value.cuda(), slots.cuda(), cache, signs.cuda())
        ref = np.full(oracle_mod.cache_shape(nb, 16, hkv, d), SENTINEL, np.uint8)
        oracle_mod.kv_write(wl.bits16(key), wl.bits16(value), "bf16", kept.numpy(), ref,
                            signs.numpy())
    elif mode == "int8":
        ik.int8_kv_write(key.cuda(), value.cuda(), slots.cuda(), cache)
        ref = np.full(oracle_mod.cache_shape_int8(nb, 16, hkv, d), SENTINEL, np.uint8)
        oracle_mod.kv_write_int8(wl.bits16(key), wl.bits16(value), "bf16", kept.numpy(), ref)
    else:
        ik.int2_kv_write(key.cuda(), value.cuda(), slots.cuda(), cache, signs.cuda())
        ref = np.full(oracle_mod.cache_shape_int2(nb, 16, hkv, d), SENTINEL, np.uint8)
        oracle_mod.kv_write_int2(wl.bits16(key), wl.bits16(value), "bf16", kept.numpy(), ref,
                                 signs.numpy())
    torch.cuda.synchronize()
    got = big.cpu().numpy()
    assert np.all(got[nb:] == SENTINEL), "a slot past the cache end was stored"
    assert np.array_equal(got[:nb], ref)


def test_decode_step_skips_slot_past_the_cache(oracle_mod):
    """The fused decode step stores a new token only when its slot lies in
    the cache; a slot in the guard blocks behind the cache is skipped."""
    header("fused decode step: a slot past the cache end is skipped")
    w = wl.custom([(1, 40), (1, 33)], 64, 8, 128, seed=17)
    nb, guard = w.num_blocks, 2
    big = torch.full(ik.cache_shape(nb + guard, 8, 128), SENTINEL, dtype=torch.uint8,
                     device="cuda")
    cache = big[:nb]
    t = to_dev(w)
    pidx, pslots = w.token_set("prior")
    ik.int4_kv_write(t["key"][pidx.cuda()], t["value"][pidx.cuda()], pslots.cuda(), cache,
                     t["signs"])
    nidx, nslots = w.token_set("new")
    nslots = nslots.clone()
    nslots[0] = nb * 16 + 5
    segs = ik.segment_buffers(2, 64, 4, 128)
    before = big.clone()
    ik.int4_decode_step(t["key"][nidx.cuda()], t["value"][nidx.cuda()], nslots.cuda(),
                        t["query"], cache, t["cu"], t["su"], 1, w.max_seqlen_k,
                        t["block_table"], w.softmax_scale, t["signs"], num_segments=4,
                        segm_output=segs[0], segm_max=segs[1], segm_expsum=segs[2])
    torch.cuda.synchronize()
    assert torch.equal(big[nb:], before[nb:]), "a slot past the cache end was stored"
    # sequence 1's new token was stored: its slot's rows changed
    s1 = int(nslots[1])
    assert not torch.equal(big[s1 // 16, :, s1 % 16], before[s1 // 16, :, s1 % 16])


@pytest.mark.gpu
@pytest.mark.parametrize("nr,nw", [(4 * 1000 + 3, 1000), (77, 300), (0, 64), (16 * 1024 * 1024 + 5, 262144)])
def test_stream_rw_definition(nr, nw):
    """The write-bandwidth comparator: written unit w is the XOR of the read
    units w, w + nw, ... below nr (16-byte units), checked on the host."""
    g = torch.Generator().manual_seed(nr * 7 + nw)
    src = torch.randint(0, 2**31 - 1, (nr * 4 + 4,), dtype=torch.int32, generator=g)
    dst = torch.full((nw * 4,), -1, dtype=torch.int32, device="cuda")
    ik.int4kv_stream_rw(src.cuda(), nr * 16, dst, nw * 16)
    units = src[: nr * 4].view(nr, 4)
    want = torch.zeros(nw, 4, dtype=torch.int32)
    for j in range((nr + nw - 1) // nw if nr else 0):
        part = units[j * nw: (j + 1) * nw]
        want[: part.shape[0]] ^= part
    assert torch.equal(dst.cpu().view(nw, 4), want)

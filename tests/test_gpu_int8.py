"""GPU parity of the INT8 per-token-head mode: the cache write (codes and
scale words bit for bit against the oracle over the whole cache buffer,
sentinel bytes included)."""
import random

import numpy as np
import pytest
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import SENTINEL, header

pytestmark = pytest.mark.gpu


def _write_both(oracle_mod, key, value, slots, nb, hkv, d, key_dev=None, value_dev=None):
    c = torch.full(ik.cache_shape_int8(nb, hkv, d), SENTINEL, dtype=torch.uint8, device="cuda")
    ik.int8_kv_write(key.cuda() if key_dev is None else key_dev,
                     value.cuda() if value_dev is None else value_dev, slots.cuda(), c)
    ref = np.full(oracle_mod.cache_shape_int8(nb, 16, hkv, d), SENTINEL, np.uint8)
    oracle_mod.kv_write_int8(wl.bits16(key), wl.bits16(value),
                             "bf16" if key.dtype == torch.bfloat16 else "f16", slots.numpy(), ref)
    torch.cuda.synchronize()
    return c.cpu().numpy(), ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hkv", [1, 4, 8])
@pytest.mark.parametrize("T", [1, 7, 42, 1000])
def test_int8_write_bit_exact(oracle_mod, T, hkv, d, dtype):
    header(f"int8 write T={T} hkv={hkv} d={d} {dtype}")
    random.seed(T + hkv + d)
    g = torch.Generator().manual_seed(T * 100 + hkv * 10 + d)
    nb = (T + 15) // 16 + 4
    slots = torch.tensor(random.sample(range(nb * 16), T), dtype=torch.int64)
    key = (2.0 * torch.randn((T, hkv, d), generator=g)).to(dtype)
    value = torch.randn((T, hkv, d), generator=g).to(dtype)
    got, ref = _write_both(oracle_mod, key, value, slots, nb, hkv, d)
    assert np.array_equal(got, ref)


def test_int8_write_ties_zero_rows_and_skips(oracle_mod):
    """Rows whose scaled values sit on exact .5 ties (absmax 127 gives scale 1),
    all-zero rows (the 1e-6 floor) and negative slots (nothing written)."""
    header("int8 write ties / zero rows / skips")
    d, T = 128, 48
    base = torch.arange(-63.5, 64.5, 1.0)[:d]  # halves: ties at scale 1
    key = torch.stack([base.clone() for _ in range(T)]).view(T, 1, d)
    key[:, 0, 0] = 127.0
    key[1::3] = 0.0
    value = -key
    slots = torch.arange(T, dtype=torch.int64) * 2
    slots[::5] = -1
    for dtype in (torch.bfloat16, torch.float16):
        got, ref = _write_both(oracle_mod, key.to(dtype), value.to(dtype), slots, 8, 1, d)
        assert np.array_equal(got, ref), dtype


def test_int8_write_strided_token_layout(oracle_mod):
    header("int8 write strided qkv")
    g = torch.Generator().manual_seed(12)
    T, hq, hkv, d = 37, 32, 8, 128
    qkv = torch.randn((T, hq + 2 * hkv, d), generator=g).to(torch.bfloat16)
    qkv_d = qkv.cuda()
    key, value = qkv[:, hq:hq + hkv], qkv[:, hq + hkv:]
    slots = torch.randperm(64 * 16, generator=g)[:T].to(torch.int64)
    got, ref = _write_both(oracle_mod, key.contiguous(), value.contiguous(), slots, 64, hkv, d,
                           key_dev=qkv_d[:, hq:hq + hkv], value_dev=qkv_d[:, hq + hkv:])
    assert np.array_equal(got, ref)


def test_int8_write_llama3_bulk_fill_sampled(oracle_mod):
    """64 x 4096 tokens, 8 KV heads, d 128, in the launch the benchmark times;
    3000 sampled tokens bit for bit, and every row written."""
    header("int8 write Llama-3-8B-shaped bulk fill (sampled)")
    w = wl.llama3_8b_decode(device="cuda")
    idx, slots = w.token_set("all")
    c = torch.full(ik.cache_shape_int8(w.num_blocks, 8, 128), SENTINEL, dtype=torch.uint8,
                   device="cuda")
    ik.int8_kv_write(w.key, w.value, slots.cuda(), c)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(2)
    pick = torch.randperm(idx.numel(), generator=g)[:3000]
    ref = np.full(oracle_mod.cache_shape_int8(w.num_blocks, 16, 8, 128), SENTINEL, np.uint8)
    oracle_mod.kv_write_int8(wl.bits16(w.key[pick.cuda()]), wl.bits16(w.value[pick.cuda()]),
                             "bf16", slots[pick].numpy(), ref)
    s = slots[pick]
    blk, off = (s // 16).numpy(), (s % 16).numpy()
    got = c.cpu().numpy()
    assert np.array_equal(got[blk, :, off], ref[blk, :, off])
    words = got[..., 128:132].copy().view("<u4")[..., 0]
    assert ((words & 0x7F800000) != 0x7F800000).all() and (words != 0xA5A5A5A5).all()

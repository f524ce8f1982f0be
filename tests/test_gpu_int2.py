"""GPU parity of the INT2 Lloyd-Max mode: the cache write (codes and scale
words bit for bit against the oracle over the whole cache buffer, sentinel
bytes included)."""
import random

import numpy as np
import pytest
import torch

import int4_quantized_paged_amd as ik
from int4_quantized_paged_amd import workloads as wl
from tests.gpu_helpers import SENTINEL, header

pytestmark = pytest.mark.gpu


def _write_both(oracle_mod, key, value, slots, nb, hkv, d, signs, key_dev=None):
    c = torch.full(ik.cache_shape_int2(nb, hkv, d), SENTINEL, dtype=torch.uint8, device="cuda")
    ik.int2_kv_write(key.cuda() if key_dev is None else key_dev, value.cuda(), slots.cuda(), c,
                     signs.cuda())
    ref = np.full(oracle_mod.cache_shape_int2(nb, 16, hkv, d), SENTINEL, np.uint8)
    oracle_mod.kv_write_int2(wl.bits16(key), wl.bits16(value),
                             "bf16" if key.dtype == torch.bfloat16 else "f16", slots.numpy(), ref,
                             signs.numpy())
    torch.cuda.synchronize()
    return c.cpu().numpy(), ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hkv", [1, 4, 8])
@pytest.mark.parametrize("T", [1, 7, 42, 1000])
def test_int2_write_bit_exact(oracle_mod, T, hkv, d, dtype):
    header(f"int2 write T={T} hkv={hkv} d={d} {dtype}")
    random.seed(T + hkv + d)
    g = torch.Generator().manual_seed(T * 100 + hkv * 10 + d)
    nb = (T + 15) // 16 + 4
    slots = torch.tensor(random.sample(range(nb * 16), T), dtype=torch.int64)
    key = (2.0 * torch.randn((T, hkv, d), generator=g)).to(dtype)
    value = torch.randn((T, hkv, d), generator=g).to(dtype)
    key[:, :, 3] *= 20.0  # an outlier channel
    got, ref = _write_both(oracle_mod, key, value, slots, nb, hkv, d, wl.rht_signs(d, seed=T))
    assert np.array_equal(got, ref)


def test_int2_write_plain_hadamard_zero_rows_skips_strides(oracle_mod):
    """All signs +1 (the unrandomised transform), all-zero rows (the 1e-6
    floor), tiny and large magnitudes, negative slots, and a key view with a
    token stride larger than its rows."""
    header("int2 write: plain Hadamard, zero rows, skips, strided key")
    d, T, hkv = 128, 64, 2
    g = torch.Generator().manual_seed(5)
    big = torch.randn((T, 2 * hkv, d), generator=g)
    big[::4] *= 1e-3
    big[1::4] *= 300.0
    big[2::9] = 0.0
    key = big[:, :hkv].to(torch.bfloat16)
    value = torch.randn((T, hkv, d), generator=g).to(torch.bfloat16)
    slots = torch.arange(T, dtype=torch.int64) * 3 % (8 * 16)
    slots[::5] = -1
    for signs in (torch.ones(d), wl.rht_signs(d, seed=3)):
        full = big.to(torch.bfloat16).cuda()
        got, ref = _write_both(oracle_mod, key, value, slots, 8, hkv, d, signs.float(),
                               key_dev=full[:, :hkv])
        assert np.array_equal(got, ref)


def test_int2_write_llama3_bulk_fill_sampled(oracle_mod):
    """The 262,144-token fill of the Llama-3-8B-shaped batch (8 KV heads,
    d 128, bf16) in one launch; 2,048 sampled tokens against the oracle."""
    w = wl.llama3_8b_decode(device="cuda")
    header(f"int2 bulk fill {w.key.shape[0]} tokens")
    c = torch.empty(ik.cache_shape_int2(w.num_blocks, 8, 128), dtype=torch.uint8, device="cuda")
    _, slots = w.token_set("all")
    signs = w.signs.cuda()
    ik.int2_kv_write(w.key, w.value, slots.cuda(), c, signs)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(1)
    pick = torch.randperm(w.key.shape[0], generator=g)[:2048]
    ref = np.zeros(oracle_mod.cache_shape_int2(w.num_blocks, 16, 8, 128), np.uint8)
    sl = slots[pick]
    oracle_mod.kv_write_int2(wl.bits16(w.key[pick.cuda()]), wl.bits16(w.value[pick.cuda()]),
                             "bf16", sl.numpy(), ref, w.signs.numpy())
    got = c.cpu().numpy()
    for s in sl.tolist():
        assert np.array_equal(got[s // 16, :, s % 16], ref[s // 16, :, s % 16]), s

"""Seeded synthetic workloads for the INT4 paged KV cache path.

This module only draws inputs: random normals, permutations, lengths, block
tables and the slot of every token.  It holds none of the method's arithmetic
(no rotation, quantization, packing or attention), so the CPU oracle and the
HIP library can both be fed from it without sharing any of the method's code.

Each workload is a batch of sequences.  Sequence ``b`` has ``kv_lens[b]`` keys;
its last ``query_lens[b]`` tokens are the queries of the attention call, and its
last ``write_lens[b]`` tokens are the tokens the timed cache write stores (the
earlier ones are "prior context", written once during set-up).

Shapes follow the pages' parameter grids and benchmark shapes:
  * tiny causal case:  1 sequence of 42 tokens, 1 KV head, head_size 64, fp16
  * GQA decode:        8 sequences of U[1, 1024] tokens, 32 q / 8 KV heads, d 128
  * Llama-3-8B-shaped decode: 64 x 4096 tokens, 32 q / 8 KV heads, K with 4
    outlier channels per head scaled by 20
  * long-context decode: 4 x 131072 tokens, 64 q / 8 KV heads, split-K
  * chunked-prefill mix: 32 sequences, query lengths log-uniform in [1, 512],
    prior contexts log-uniform in [512, 16384], d 128 or 64
Random numbers come from ``torch.Generator`` seeded per workload.  Normals are
drawn in fp32 and rounded to the 16-bit input dtype.  Large workloads may be
drawn on the GPU (``device="cuda"``); the stream then differs from the CPU one
but stays seeded and reproducible on the same software stack.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK_SIZE = 16


def rht_signs(head_size: int, seed: int = 0) -> torch.Tensor:
    """Sign vector of the random Hadamard rotation: +-1.0 Bernoulli(0.5), fp32."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randint(0, 2, (head_size,), generator=g) * 2 - 1).to(torch.float32)


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    num_blocks: int
    kv_lens: list[int]
    query_lens: list[int]
    write_lens: list[int]
    block_table: torch.Tensor          # int32 [S, max_blocks_per_seq]
    key: torch.Tensor                  # [sum(kv_lens), Hkv, d] every token of every sequence
    value: torch.Tensor
    query: torch.Tensor                # [sum(query_lens), Hq, d]
    signs: torch.Tensor                # fp32 [d]
    block_size: int = BLOCK_SIZE
    notes: dict = field(default_factory=dict)

    # ---- derived metadata (plain bookkeeping) ----
    @property
    def num_seqs(self) -> int:
        return len(self.kv_lens)

    @property
    def softmax_scale(self) -> float:
        return self.head_size ** -0.5

    @property
    def max_seqlen_q(self) -> int:
        return max(self.query_lens) if self.query_lens else 0

    @property
    def max_seqlen_k(self) -> int:
        return max(self.kv_lens) if self.kv_lens else 0

    def cu_seqlens_q(self) -> torch.Tensor:
        c = [0]
        for q in self.query_lens:
            c.append(c[-1] + q)
        return torch.tensor(c, dtype=torch.int32)

    def seqused_k(self) -> torch.Tensor:
        return torch.tensor(self.kv_lens, dtype=torch.int32)

    def token_offsets(self) -> list[int]:
        off = [0]
        for L in self.kv_lens:
            off.append(off[-1] + L)
        return off

    def slots_of(self, b: int, positions: torch.Tensor) -> torch.Tensor:
        """slot = block_table[b, pos // block_size] * block_size + pos % block_size."""
        bt = self.block_table[b].to(torch.int64).to(positions.device)
        return bt[positions // self.block_size] * self.block_size + positions % self.block_size

    def token_set(self, which: str):
        """Global token indices and slots: which = "prior" | "new" | "all"."""
        idx, slots = [], []
        off = self.token_offsets()
        for b, L in enumerate(self.kv_lens):
            w = self.write_lens[b]
            lo, hi = {"prior": (0, L - w), "new": (L - w, L), "all": (0, L)}[which]
            if hi <= lo:
                continue
            pos = torch.arange(lo, hi, dtype=torch.int64)
            idx.append(pos + off[b])
            slots.append(self.slots_of(b, pos))
        if not idx:
            e = torch.zeros(0, dtype=torch.int64)
            return e, e
        return torch.cat(idx), torch.cat(slots)

    def kv_bytes_attended(self) -> int:
        """Packed K+V bytes a causal pass must read: one row per (key, KV head).

        Query i of sequence b sees keys [0, L_b - q_b + i]; the longest row of
        the sequence (its last query) covers all L_b keys, and a kernel that
        shares K/V tiles across the rows of a sequence reads each key once."""
        R = self.head_size // 2 + 4
        return sum(self.kv_lens) * self.num_kv_heads * 2 * R

    def attention_flops(self) -> int:
        """Algorithmic flops of causal attention: 2*d for Q.K and 2*d for P.V
        per (query row, visible key, query head).  Query i of sequence b sees
        L_b - q_b + i + 1 keys."""
        pairs = 0
        for L, q in zip(self.kv_lens, self.query_lens):
            pairs += q * (L - q) + q * (q + 1) // 2
        return pairs * self.num_q_heads * 4 * self.head_size

    def write_bytes(self, which: str = "new") -> int:
        """Algorithmic bytes of the cache write: K and V inputs read, packed
        rows written, one int64 slot per token."""
        idx, _ = self.token_set(which)
        T = int(idx.numel())
        esz = torch.finfo(self.dtype).bits // 8
        R = self.head_size // 2 + 4
        return T * (self.num_kv_heads * (2 * self.head_size * esz + 2 * R) + 8)


def _normal(shape, gen, dtype, device):
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device).to(dtype)


def _gen(seed: int, device) -> torch.Generator:
    return torch.Generator(device=device).manual_seed(seed)


def tiny(device="cpu") -> Workload:
    """One sequence of 42 tokens, 1 KV head, 1 query head, d 64, fp16, seed 0.
    Identity block table over 3 blocks; all 42 tokens are written, then one
    decode query at position 41."""
    g = _gen(0, device)
    d, T = 64, 42
    key = _normal((T, 1, d), g, torch.float16, device)
    value = _normal((T, 1, d), g, torch.float16, device)
    query = _normal((1, 1, d), g, torch.float16, device)
    return Workload("tiny causal 1x42 d64 fp16", torch.float16, 1, 1, d, 3, [T], [1], [T],
                    torch.tensor([[0, 1, 2]], dtype=torch.int32), key, value, query,
                    rht_signs(d))


def _disjoint_tables(nblocks_per_seq: list[int], num_blocks: int, g_cpu) -> torch.Tensor:
    perm = torch.randperm(num_blocks, generator=g_cpu).to(torch.int32)
    width = max(nblocks_per_seq) if nblocks_per_seq else 1
    bt = torch.zeros((len(nblocks_per_seq), width), dtype=torch.int32)
    o = 0
    for b, n in enumerate(nblocks_per_seq):
        bt[b, :n] = perm[o:o + n]
        o += n
    return bt


def gqa_decode(device="cpu", seed: int = 1) -> Workload:
    """8 sequences with lengths uniform in [1, 1024], 32 q / 8 KV heads, d 128,
    bf16, 1024-block pool; sequence b owns blocks perm[64b : 64b + 64].  One new
    token per sequence is written, then one decode step."""
    gc = torch.Generator().manual_seed(seed)
    S, Hq, Hkv, d, NB = 8, 32, 8, 128, 1024
    kv_lens = torch.randint(1, 1025, (S,), generator=gc).tolist()
    perm = torch.randperm(NB, generator=gc).to(torch.int32)
    bt = perm[:S * 64].view(S, 64).clone()
    g = gc if str(device) == "cpu" else _gen(seed, device)
    N = sum(kv_lens)
    key = _normal((N, Hkv, d), g, torch.bfloat16, device)
    value = _normal((N, Hkv, d), g, torch.bfloat16, device)
    query = _normal((S, Hq, d), g, torch.bfloat16, device)
    return Workload("GQA decode 8xU[1,1024] 32q/8kv d128 bf16", torch.bfloat16, Hq, Hkv, d, NB,
                    kv_lens, [1] * S, [1] * S, bt, key, value, query, rht_signs(d))


def llama3_8b_decode(device="cpu", seed: int = 2, num_seqs: int = 64,
                     ctx: int = 4096) -> Workload:
    """Llama-3-8B-shaped decode: 64 sequences x 4096 tokens, 32 q / 8 KV heads,
    d 128, bf16.  K is N(0,1) except 4 fixed outlier channels per KV head that
    are scaled by 20; V and Q are N(0,1).  Random block table over a pool sized
    for the whole batch."""
    gc = torch.Generator().manual_seed(seed)
    S, Hq, Hkv, d = num_seqs, 32, 8, 128
    nbs = ctx // BLOCK_SIZE
    NB = S * nbs
    bt = torch.randperm(NB, generator=gc).to(torch.int32).view(S, nbs).clone()
    outliers = torch.stack([torch.randperm(d, generator=gc)[:4] for _ in range(Hkv)])
    g = gc if str(device) == "cpu" else _gen(seed, device)
    N = S * ctx
    kf = torch.randn((N, Hkv, d), generator=g, dtype=torch.float32, device=device)
    for h in range(Hkv):
        kf[:, h, outliers[h].to(kf.device)] *= 20.0
    key = kf.to(torch.bfloat16)
    del kf
    value = _normal((N, Hkv, d), g, torch.bfloat16, device)
    query = _normal((S, Hq, d), g, torch.bfloat16, device)
    return Workload(f"Llama-3-8B-shaped decode {S}x{ctx} 32q/8kv d128 bf16", torch.bfloat16,
                    Hq, Hkv, d, NB, [ctx] * S, [1] * S, [1] * S, bt, key, value, query,
                    rht_signs(d), notes={"outlier_channels": outliers})


def long_context_decode(device="cpu", seed: int = 3, num_seqs: int = 4,
                        ctx: int = 131072) -> Workload:
    """Long-context decode: 4 sequences x 131072 tokens, 64 q / 8 KV heads (G=8),
    d 128, bf16 N(0,1) K/V/Q, random block table; decoded with split-K."""
    gc = torch.Generator().manual_seed(seed)
    S, Hq, Hkv, d = num_seqs, 64, 8, 128
    nbs = ctx // BLOCK_SIZE
    NB = S * nbs
    bt = torch.randperm(NB, generator=gc).to(torch.int32).view(S, nbs).clone()
    g = gc if str(device) == "cpu" else _gen(seed, device)
    N = S * ctx
    key = _normal((N, Hkv, d), g, torch.bfloat16, device)
    value = _normal((N, Hkv, d), g, torch.bfloat16, device)
    query = _normal((S, Hq, d), g, torch.bfloat16, device)
    return Workload(f"long-context decode {S}x{ctx} 64q/8kv d128 bf16", torch.bfloat16, Hq, Hkv,
                    d, NB, [ctx] * S, [1] * S, [1] * S, bt, key, value, query, rht_signs(d))


def serving_standin(device="cpu", seed: int = 5) -> Workload:
    """Serving stand-in: 100 sequences whose 512-token prompts are written,
    then one decode step each at a context uniform in [512, 640] (its last key
    is the step's new token; the keys between the prompt and it are written
    beforehand); 32 q / 8 KV heads, d 128, bf16 N(0,1), disjoint random
    blocks."""
    gc = torch.Generator().manual_seed(seed)
    S, Hq, Hkv, d = 100, 32, 8, 128
    kv_lens = torch.randint(512, 641, (S,), generator=gc).tolist()
    nbl = [(L + BLOCK_SIZE - 1) // BLOCK_SIZE for L in kv_lens]
    NB = sum(nbl)
    bt = _disjoint_tables(nbl, NB, gc)
    g = gc if str(device) == "cpu" else _gen(seed, device)
    N = sum(kv_lens)
    key = _normal((N, Hkv, d), g, torch.bfloat16, device)
    value = _normal((N, Hkv, d), g, torch.bfloat16, device)
    query = _normal((S, Hq, d), g, torch.bfloat16, device)
    return Workload("serving stand-in 100x512 prompts, decode at 512..640 32q/8kv d128 bf16",
                    torch.bfloat16, Hq, Hkv, d, NB, kv_lens, [1] * S, [1] * S, bt, key, value,
                    query, rht_signs(d))


def chunked_prefill(device="cpu", seed: int = 4, head_size: int = 128,
                    num_seqs: int = 32) -> Workload:
    """Chunked-prefill mixed batch: 32 sequences, query lengths
    clamp(round(exp(U(0, ln 512))), 1, 512), prior contexts
    clamp(round(exp(U(ln 512, ln 16384))), 512, 16384); 32 q / 8 KV heads, bf16.
    The new tokens are written, then causal attention over the full context."""
    gc = torch.Generator().manual_seed(seed)
    S, Hq, Hkv, d = num_seqs, 32, 8, head_size
    u1 = torch.rand(S, generator=gc, dtype=torch.float64)
    u2 = torch.rand(S, generator=gc, dtype=torch.float64)
    q_lens = [int(min(max(round(math.exp(x * math.log(512))), 1), 512)) for x in u1.tolist()]
    ctxs = [int(min(max(round(math.exp(math.log(512) + x * (math.log(16384) - math.log(512)))),
                        512), 16384)) for x in u2.tolist()]
    kv_lens = [c + q for c, q in zip(ctxs, q_lens)]
    nbl = [(L + BLOCK_SIZE - 1) // BLOCK_SIZE for L in kv_lens]
    NB = sum(nbl)
    bt = _disjoint_tables(nbl, NB, gc)
    g = gc if str(device) == "cpu" else _gen(seed, device)
    N = sum(kv_lens)
    key = _normal((N, Hkv, d), g, torch.bfloat16, device)
    value = _normal((N, Hkv, d), g, torch.bfloat16, device)
    query = _normal((sum(q_lens), Hq, d), g, torch.bfloat16, device)
    return Workload(f"chunked-prefill mix {S} seqs 32q/8kv d{d} bf16", torch.bfloat16, Hq, Hkv,
                    d, NB, kv_lens, q_lens, list(q_lens), bt, key, value, query, rht_signs(d))


def custom(num_seqs_lens: list[tuple[int, int]], num_q_heads: int, num_kv_heads: int,
           head_size: int, dtype=torch.bfloat16, seed: int = 0, device="cpu",
           write_all: bool = False, extra_blocks: int = 0, scale: float = 1.0) -> Workload:
    """Small ad-hoc batch: ``num_seqs_lens`` = [(query_len, kv_len), ...].
    Disjoint random block tables; prior context is every token before the
    queries unless ``write_all``."""
    gc = torch.Generator().manual_seed(seed)
    q_lens = [q for q, _ in num_seqs_lens]
    kv_lens = [k for _, k in num_seqs_lens]
    nbl = [max(1, (L + BLOCK_SIZE - 1) // BLOCK_SIZE) for L in kv_lens]
    NB = sum(nbl) + extra_blocks
    bt = _disjoint_tables(nbl, NB, gc)
    g = gc if str(device) == "cpu" else _gen(seed, device)
    N = sum(kv_lens)
    key = (torch.randn((N, num_kv_heads, head_size), generator=g, device=device) * scale).to(dtype)
    value = (torch.randn((N, num_kv_heads, head_size), generator=g, device=device) * scale).to(dtype)
    query = torch.randn((sum(q_lens), num_q_heads, head_size), generator=g,
                        device=device).to(dtype)
    w = list(kv_lens) if write_all else list(q_lens)
    return Workload(f"custom {num_seqs_lens} {num_q_heads}q/{num_kv_heads}kv d{head_size}",
                    dtype, num_q_heads, num_kv_heads, head_size, NB, kv_lens, q_lens, w, bt,
                    key, value, query, rht_signs(head_size))


def bits16(t: torch.Tensor):
    """Raw 16-bit patterns of an fp16/bf16 tensor as a numpy uint16 array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")

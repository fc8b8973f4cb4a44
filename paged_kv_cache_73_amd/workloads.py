"""Seeded synthetic workloads shaped like the paged-attention examples.

This module only draws inputs: sequence lengths, the order in which physical block
ids are handed out, and normally distributed q/K/V values rounded to the storage
dtype.  It contains no attention arithmetic and no block-table arithmetic: block
tables, slot mappings and packed-batch offsets are built from these inputs by the
block manager under test (the library's C++ one, or the oracle's own).

Geometry is Qwen3-0.6B's attention layer (16 query heads, 8 KV heads, head_dim 128,
bf16) unless stated otherwise, as in "从零开始写Qwen3（六）PagedAttention",
KVCache大小计算.  Random streams: ``random.Random(seed)`` for lengths and the block
order, ``torch.Generator().manual_seed(seed)`` for tensor values, drawn on the CPU
so every machine sees the same bits.
"""

from __future__ import annotations

import math
import random
from dataclasses import dataclass, field

import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "bf16": 2}


def _randn(shape, gen: torch.Generator, dtype: str) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(TORCH_DTYPES[dtype])


def _blocks_for(tokens: int, block_size: int) -> int:
    return (tokens + block_size - 1) // block_size


@dataclass
class Workload:
    """Inputs of one paged-attention workload.

    ``cached[b]`` tokens of sequence b are already in the cache (values ``k_ctx`` /
    ``v_ctx``, concatenated over sequences in order); ``new[b]`` tokens are appended
    by the step (values ``k_new`` / ``v_new``, concatenated likewise) at positions
    cached[b] .. cached[b]+new[b]-1.  Decode workloads have new[b] == 1 and one
    query per sequence; prefill workloads have one query per new token.

    ``groups`` (shared-prefix workloads only) lists, per group, the member sequence
    indices; the first ``prefix_len`` tokens of every member are the same physical
    blocks, and ``snapshot_last`` asks for one extra holder of each member's last
    partial block so that the append must copy it first.
    """

    name: str
    kind: str                    # "decode" or "prefill"
    dtype: str                   # "f32" or "bf16"
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks: int              # block-table width
    cached: list[int]
    new: list[int]
    order: list[int]             # physical ids in the order the free stack hands them out
    q: torch.Tensor              # decode [batch, Hq, d]; prefill [sum(new), Hq, d]
    k_ctx: torch.Tensor          # [sum(cached) or prefix-deduplicated, Hkv, d]
    v_ctx: torch.Tensor
    k_new: torch.Tensor          # [sum(new), Hkv, d]
    v_new: torch.Tensor
    scale: float
    causal: bool = True
    groups: list[list[int]] | None = None
    prefix_len: int = 0
    snapshot_last: bool = False
    seed: int = 0
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.cached)

    @property
    def seqlens_k(self) -> list[int]:
        return [c + n for c, n in zip(self.cached, self.new)]

    @property
    def kv_dim(self) -> int:
        return self.num_kv_heads * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


def _finish(name, kind, dtype, hq, hkv, d, bs, cached, new, num_blocks, max_blocks, rng, gen,
            scale=None, ctx_tokens=None, **kw) -> Workload:
    order = list(range(num_blocks))
    rng.shuffle(order)
    ctx_tokens = sum(cached) if ctx_tokens is None else ctx_tokens
    n_new = sum(new)
    n_q = len(cached) if kind == "decode" else n_new
    k_ctx = _randn((ctx_tokens, hkv, d), gen, dtype)
    v_ctx = _randn((ctx_tokens, hkv, d), gen, dtype)
    k_new = _randn((n_new, hkv, d), gen, dtype)
    v_new = _randn((n_new, hkv, d), gen, dtype)
    q = _randn((n_q, hq, d), gen, dtype)
    return Workload(name=name, kind=kind, dtype=dtype, num_heads=hq, num_kv_heads=hkv,
                    head_dim=d, block_size=bs, num_blocks=num_blocks, max_blocks=max_blocks,
                    cached=list(cached), new=list(new), order=order, q=q, k_ctx=k_ctx,
                    v_ctx=v_ctx, k_new=k_new, v_new=v_new,
                    scale=scale if scale is not None else 1.0 / math.sqrt(d), **kw)


def _pool_for(need_blocks: int, slack: float) -> int:
    return int(math.ceil(slack * need_blocks))


def decode_workload(cached, *, dtype="bf16", num_heads=16, num_kv_heads=8, head_dim=128,
                    block_size=16, num_blocks=None, max_blocks=None, slack=1.1, seed=0,
                    name="decode") -> Workload:
    """One new token per sequence, appended at position cached[b], then a decode over
    cached[b] + 1 keys."""
    rng = random.Random(seed)
    gen = torch.Generator().manual_seed(seed)
    cached = [int(c) for c in cached]
    seqlens = [c + 1 for c in cached]
    need = sum(_blocks_for(s, block_size) for s in seqlens)
    width = max(_blocks_for(s, block_size) for s in seqlens)
    num_blocks = _pool_for(need, slack) if num_blocks is None else num_blocks
    max_blocks = width if max_blocks is None else max_blocks
    return _finish(name, "decode", dtype, num_heads, num_kv_heads, head_dim, block_size,
                   cached, [1] * len(cached), num_blocks, max_blocks, rng, gen, seed=seed)


def prefill_workload(cached, new, *, dtype="bf16", num_heads=16, num_kv_heads=8,
                     head_dim=128, block_size=16, num_blocks=None, max_blocks=None,
                     slack=1.1, causal=True, seed=0, name="prefill") -> Workload:
    """Chunked prefill: new[i] query tokens appended after cached[i] cached tokens."""
    rng = random.Random(seed)
    gen = torch.Generator().manual_seed(seed)
    seqlens = [c + n for c, n in zip(cached, new)]
    need = sum(_blocks_for(s, block_size) for s in seqlens)
    width = max([_blocks_for(s, block_size) for s in seqlens] + [1])
    num_blocks = max(1, _pool_for(need, slack)) if num_blocks is None else num_blocks
    max_blocks = width if max_blocks is None else max_blocks
    return _finish(name, "prefill", dtype, num_heads, num_kv_heads, head_dim, block_size,
                   list(cached), list(new), num_blocks, max_blocks, rng, gen,
                   causal=causal, seed=seed)


# --------------------------------------------------------------------------------------
# the named workloads
# --------------------------------------------------------------------------------------

def tiny_decode(seed: int = 0) -> Workload:
    """Tiny fp32 decode shaped like the decode example of "Sayfalı dikkat" (Çözme yolu):
    cache_seqlens [30, 32, 70], block size 32, at most 4 blocks per sequence, a pool
    of 16 blocks handed out in a seeded random order; 4 query / 2 KV heads, d = 64."""
    return decode_workload([30, 32, 70], dtype="f32", num_heads=4, num_kv_heads=2,
                           head_dim=64, block_size=32, num_blocks=16, max_blocks=4,
                           seed=seed, name="tiny_decode_f32")


def qwen3_decode(seed: int = 0, batch: int = 64, lo: int = 512, hi: int = 4096) -> Workload:
    """Single-layer decode at Qwen3-0.6B shape: batch 64, context lengths uniform in
    [512, 4096] (the appended token included), block size 16, pool = need + 10 %."""
    rng = random.Random(seed ^ 0x5EED)
    ctx = [rng.randint(lo, hi) for _ in range(batch)]
    return decode_workload([c - 1 for c in ctx], seed=seed, name="qwen3_decode_b64")


def gqa8_decode(seed: int = 0, batch: int = 64, lo: int = 512, hi: int = 4096) -> Workload:
    """Decode with eight query heads per KV head (64 query / 8 KV heads, head_dim 128):
    batch 64, contexts uniform in [512, 4096], block size 16.  In bf16 this group size
    runs on the matrix-core route."""
    rng = random.Random(seed ^ 0x5EED)
    ctx = [rng.randint(lo, hi) for _ in range(batch)]
    return decode_workload([c - 1 for c in ctx], seed=seed, num_heads=64, num_kv_heads=8,
                           head_dim=128, block_size=16, name="gqa8_decode_b64")


def long_decode(seed: int = 0, batch: int = 8, lo: int = 32768, hi: int = 40960) -> Workload:
    """Long-context decode: batch 8, contexts uniform in [32768, 40960] (up to the 40K
    maximum length of Qwen3-0.6B); the split-K partition size is a call argument."""
    rng = random.Random(seed ^ 0x5EED)
    ctx = [rng.randint(lo, hi) for _ in range(batch)]
    return decode_workload([c - 1 for c in ctx], seed=seed, name="long_decode_b8")


def shared_prefix_decode(seed: int = 0, groups: int = 4, per_group: int = 32,
                         prefix_len: int = 2048, suffix_lo: int = 64,
                         suffix_hi: int = 512, block_size: int = 16) -> Workload:
    """Shared-prefix decode: ``groups`` groups of ``per_group`` sequences; members of a
    group share the physical blocks of a ``prefix_len``-token prefix and own a private
    suffix of suffix_lo..suffix_hi tokens whose length is not a multiple of the block
    size.  An extra holder keeps a reference on each member's last (partial) block, so
    the append copies it first (copy-on-write).  ``k_ctx`` holds each group's prefix
    once, followed by every member's suffix."""
    rng = random.Random(seed ^ 0x5EED)
    gen = torch.Generator().manual_seed(seed)
    suffixes = []
    for _ in range(groups * per_group):
        s = rng.randint(suffix_lo, suffix_hi)
        while s % block_size == 0:
            s = rng.randint(suffix_lo, suffix_hi)
        suffixes.append(s)
    cached = [prefix_len + s for s in suffixes]
    members = [list(range(g * per_group, (g + 1) * per_group)) for g in range(groups)]
    prefix_blocks = _blocks_for(prefix_len, block_size)
    # prefix blocks once per group, private blocks per member (+1 copy-on-write target)
    need = groups * prefix_blocks + sum(_blocks_for(prefix_len + s + 1, block_size) - prefix_blocks + 1
                                        for s in suffixes)
    num_blocks = _pool_for(need, 1.1)
    max_blocks = max(_blocks_for(c + 1, block_size) for c in cached)
    ctx_tokens = groups * prefix_len + sum(suffixes)
    return _finish("shared_prefix_decode_b128", "decode", "bf16", 16, 8, 128, block_size,
                   cached, [1] * len(cached), num_blocks, max_blocks, rng, gen,
                   ctx_tokens=ctx_tokens, groups=members, prefix_len=prefix_len,
                   snapshot_last=True, seed=seed)


def chunked_prefill(seed: int = 0, batch: int = 16, q_hi: int = 512, c_hi: int = 4096) -> Workload:
    """Chunked prefill: 16 requests, query lengths uniform in [1, 512], cached lengths
    uniform in [0, 4096], causal, Qwen3-0.6B geometry, block size 16."""
    rng = random.Random(seed ^ 0x5EED)
    new = [rng.randint(1, q_hi) for _ in range(batch)]
    cached = [rng.randint(0, c_hi) for _ in range(batch)]
    return prefill_workload(cached, new, seed=seed, name="chunked_prefill_r16")


def contiguous_kv(w: Workload) -> tuple[torch.Tensor, torch.Tensor]:
    """The workload's keys and values packed per request, without a cache: request b's
    cached rows followed by its new rows, requests in order, ``[sum(seqlens_k), Hkv,
    d]`` each.  (Shared-prefix workloads store a prefix once and have no such form.)"""
    if w.groups is not None:
        raise ValueError("a shared-prefix workload has no contiguous form")
    ks, vs, c0, n0 = [], [], 0, 0
    for c, n in zip(w.cached, w.new):
        ks += [w.k_ctx[c0:c0 + c], w.k_new[n0:n0 + n]]
        vs += [w.v_ctx[c0:c0 + c], w.v_new[n0:n0 + n]]
        c0, n0 = c0 + c, n0 + n
    return torch.cat(ks).contiguous(), torch.cat(vs).contiguous()


# --------------------------------------------------------------------------------------
# driving a block manager through a workload
# --------------------------------------------------------------------------------------

@dataclass
class Plan:
    """Host metadata of a workload, produced by one block manager and its builders."""

    tables: list[list[int]]       # [batch][max_blocks], -1 = unassigned
    ctx_slots: list[int]          # slot of every k_ctx / v_ctx row
    copies: list[tuple[int, int]] # copy-on-write pairs of the step, in order
    new_slots: list[int]          # slot of every k_new / v_new row
    seqlens_k: list[int]
    cu_q: list[int]
    cu_k: list[int]
    max_q: int
    max_k: int
    manager: object = None


def plan(w: Workload, manager_cls, slot_mapping, cu_seqlens) -> Plan:
    """Replay the workload's block-manager calls on ``manager_cls`` and build the
    metadata with the given builders.  The same sequence of calls is made whichever
    implementation is passed (the library's or the oracle's); only they compute.

    Context: every sequence's cached tokens get blocks (shared-prefix workloads take the
    group's prefix blocks once, then share them with every member and release the
    founding row).  Step: the new tokens' positions are made writable, which allocates
    a block when a sequence crosses a block boundary and copies a shared block first.
    """
    B = w.block_size
    bm = manager_cls(w.num_blocks, initial_order=w.order)
    rows = [[-1] * w.max_blocks for _ in range(w.batch)]
    ctx_seq, ctx_pos = [], []
    if w.groups is None:
        for b in range(w.batch):
            bm.prepare_write(rows[b], 0, w.cached[b], B)
            ctx_seq += [b] * w.cached[b]
            ctx_pos += list(range(w.cached[b]))
    else:
        for members in w.groups:
            base = [-1] * w.max_blocks
            bm.prepare_write(base, 0, w.prefix_len, B)
            for b in members:
                rows[b] = bm.share(base)
            bm.release_table(base)
            ctx_seq += [members[0]] * w.prefix_len
            ctx_pos += list(range(w.prefix_len))
        for members in w.groups:
            for b in members:
                bm.prepare_write(rows[b], w.prefix_len, w.cached[b] - w.prefix_len, B)
                ctx_seq += [b] * (w.cached[b] - w.prefix_len)
                ctx_pos += list(range(w.prefix_len, w.cached[b]))
        if w.snapshot_last:
            for b in range(w.batch):
                bm.incref(rows[b][(w.cached[b] - 1) // B])
    ctx_slots = [int(x) for x in slot_mapping(rows, B, ctx_seq, ctx_pos)] if ctx_seq else []
    copies = []
    new_seq, new_pos = [], []
    for b in range(w.batch):
        copies += bm.prepare_write(rows[b], w.cached[b], w.new[b], B)
        new_seq += [b] * w.new[b]
        new_pos += list(range(w.cached[b], w.cached[b] + w.new[b]))
    new_slots = [int(x) for x in slot_mapping(rows, B, new_seq, new_pos)] if new_seq else []
    seqlens = w.seqlens_k
    cu_q, max_q = cu_seqlens(w.new)
    cu_k, max_k = cu_seqlens(seqlens)
    return Plan(tables=[list(map(int, r)) for r in rows], ctx_slots=ctx_slots,
                copies=[(int(s), int(d)) for s, d in copies], new_slots=new_slots,
                seqlens_k=list(seqlens), cu_q=[int(x) for x in cu_q], cu_k=[int(x) for x in cu_k],
                max_q=int(max_q), max_k=int(max_k), manager=bm)

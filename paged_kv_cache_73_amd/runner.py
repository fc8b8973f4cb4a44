"""Puts a synthetic workload on the device through libpa and runs its step.

Set-up (not part of a step): the library's block manager plans the tables and slots,
the pools are filled with NaN, and the cached context is written with pa_write_kv.
A step is the hot path of one layer: pa_copy_blocks for the copy-on-write pairs (if
any), pa_write_kv for the new tokens, then pa_decode or pa_prefill_varlen.  A fused
decode step replaces the last two by pa_decode_append.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import _native as pa
from . import workloads as W


@dataclass
class DeviceRun:
    plan: W.Plan
    pool: pa.KVPool
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    q: torch.Tensor
    out: torch.Tensor
    table: torch.Tensor
    seqlens: torch.Tensor
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    new_slots: torch.Tensor
    k_new: torch.Tensor
    v_new: torch.Tensor
    copy_src: torch.Tensor
    copy_dst: torch.Tensor
    workspace: torch.Tensor | None = None
    prefill_ws: torch.Tensor | None = None


def _i32(x, dev) -> torch.Tensor:
    arr = np.asarray(x, dtype=np.int32).reshape(-1) if len(x) else np.zeros(0, np.int32)
    return torch.tensor(arr, dtype=torch.int32, device=dev)


def setup(w: W.Workload, dev="cuda") -> DeviceRun:
    p = W.plan(w, pa.BlockManager, pa.pa_build_slot_mapping, pa.pa_build_cu_seqlens)
    tdt = W.TORCH_DTYPES[w.dtype]
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kc = torch.full(shape, float("nan"), dtype=tdt, device=dev)
    vc = torch.full(shape, float("nan"), dtype=tdt, device=dev)
    pool = pa.KVPool(kc, vc)
    if p.ctx_slots:
        pa.pa_write_kv(pool, w.k_ctx.to(dev), w.v_ctx.to(dev), _i32(p.ctx_slots, dev))
    table = torch.tensor(np.asarray(p.tables, dtype=np.int32), device=dev)
    out = torch.zeros(w.q.shape, dtype=tdt, device=dev)
    return DeviceRun(plan=p, pool=pool, k_cache=kc, v_cache=vc, q=w.q.to(dev), out=out,
                     table=table, seqlens=_i32(p.seqlens_k, dev), cu_q=_i32(p.cu_q, dev),
                     cu_k=_i32(p.cu_k, dev), new_slots=_i32(p.new_slots, dev),
                     k_new=w.k_new.to(dev), v_new=w.v_new.to(dev),
                     copy_src=_i32([s for s, _ in p.copies], dev),
                     copy_dst=_i32([d for _, d in p.copies], dev))


def ensure_workspace(w: W.Workload, r: DeviceRun, partition_tokens: int) -> None:
    max_k = max(r.plan.seqlens_k) if r.plan.seqlens_k else 0
    ws = pa.pa_decode_workspace_bytes(w.batch, w.num_heads, w.num_kv_heads, w.head_dim, max_k,
                                      partition_tokens, w.block_size)
    if r.workspace is None or r.workspace.numel() < ws:
        r.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=r.q.device)


def write(w: W.Workload, r: DeviceRun) -> None:
    """Copy-on-write copies, then the KV write of the step's new tokens."""
    if r.copy_src.numel():
        pa.pa_copy_blocks(r.pool, r.copy_src, r.copy_dst)
    pa.pa_write_kv(r.pool, r.k_new, r.v_new, r.new_slots)


def attend(w: W.Workload, r: DeviceRun, partition_tokens: int = 0) -> None:
    if w.kind == "decode":
        ensure_workspace(w, r, partition_tokens)
        max_k = max(r.plan.seqlens_k) if r.plan.seqlens_k else 0
        pa.pa_decode(r.pool, r.out, r.q, r.table, r.seqlens, max_k, w.scale, partition_tokens,
                     r.workspace)
    else:
        pa.pa_prefill_varlen(r.pool, r.out, r.q, r.cu_q, r.cu_k, r.plan.max_q, r.plan.max_k,
                             r.table, w.scale, w.causal)


def attend_splitk(w: W.Workload, r: DeviceRun) -> None:
    """The prefill with key splitting (pa_prefill_varlen_splitk), planned from host copies
    of the lengths; the workspace is sized once per run."""
    hq, hk = r.plan.cu_q, r.plan.cu_k
    if r.prefill_ws is None:
        dt = pa.PA_BF16 if w.dtype == "bf16" else pa.PA_F32
        need = pa.pa_prefill_workspace_bytes(dt, w.batch, w.num_heads, w.num_kv_heads,
                                             w.head_dim, w.block_size, r.plan.max_q,
                                             r.plan.max_k, w.causal, hq, hk)
        r.prefill_ws = torch.empty(max(need, 1), dtype=torch.uint8, device=r.q.device)
    pa.pa_prefill_varlen_splitk(r.pool, r.out, r.q, r.cu_q, r.cu_k, r.plan.max_q, r.plan.max_k,
                                r.table, w.scale, w.causal, r.prefill_ws, hq, hk)


def attend_contiguous(w: W.Workload, r: DeviceRun, k: torch.Tensor, v: torch.Tensor) -> None:
    """The prefill over packed contiguous K/V (no block table)."""
    pa.pa_prefill_varlen_contiguous(r.out, r.q, k, v, r.cu_q, r.cu_k, r.plan.max_q, r.plan.max_k,
                                    w.scale, w.causal)


def attend_partials(w: W.Workload, r: DeviceRun, partition_tokens: int = 0) -> None:
    """Pass 1 of the decode (pa_decode_partials); attend_merge completes it."""
    ensure_workspace(w, r, partition_tokens)
    max_k = max(r.plan.seqlens_k) if r.plan.seqlens_k else 0
    pa.pa_decode_partials(r.pool, r.out, r.q, r.table, r.seqlens, max_k, w.scale,
                          partition_tokens, r.workspace)


def attend_merge(w: W.Workload, r: DeviceRun, partition_tokens: int = 0) -> None:
    """Pass 2 of the decode (pa_decode_merge)."""
    max_k = max(r.plan.seqlens_k) if r.plan.seqlens_k else 0
    pa.pa_decode_merge(r.pool, r.out, r.table, r.seqlens, max_k, partition_tokens, r.workspace)


def attend_append(w: W.Workload, r: DeviceRun, partition_tokens: int = 0) -> None:
    """Decode with the new tokens' K/V stored by the attention launch itself."""
    if w.kind != "decode":
        raise ValueError("the fused append is a decode step")
    ensure_workspace(w, r, partition_tokens)
    max_k = max(r.plan.seqlens_k) if r.plan.seqlens_k else 0
    pa.pa_decode_append(r.pool, r.out, r.q, r.k_new, r.v_new, r.table, r.seqlens, max_k,
                        w.scale, partition_tokens, r.workspace)


def step(w: W.Workload, r: DeviceRun, partition_tokens: int = 0, attention: bool = True,
         fused: bool = False) -> None:
    if fused:
        if r.copy_src.numel():
            pa.pa_copy_blocks(r.pool, r.copy_src, r.copy_dst)
        attend_append(w, r, partition_tokens)
        return
    write(w, r)
    if attention:
        attend(w, r, partition_tokens)

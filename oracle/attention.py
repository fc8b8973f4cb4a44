"""Oracle for the KV write, the paged index, and decode / varlen-prefill attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Float64 throughout; bf16
values are decoded by this module's own codec.  Storage arrays are passed as raw
numpy arrays: ``uint16`` holding bf16 bit patterns, or ``float32``.

Pins (tests/test_oracle_pins.py):
  * online_softmax_trace   -- printed trace of 题目2 and its closed form.
  * flash_tiles            -- printed m, l and correction factors of 题目3, plus the
                              closed-form dense result for the lost final O.
  * copy_blocks            -- pools whose every element encodes its own position:
                              destination blocks hold exactly the source blocks'
                              codes in K and in V, every other block is untouched,
                              an empty pair list is a no-op.
  * locate / element_offset-- 题目5 (table [3,1,5]) and the Sayfalı dikkat decode
                              example (cache_seqlens [30,32,70], B=32).
  * gather / decode        -- brute-force dense attention on the un-paged values,
                              single-key, zero-query and MHA special cases.
  * prefill_varlen         -- equal to decode for q_len = 1; chunked prefill equals
                              one-shot prefill row by row; the non-causal last row
                              equals dense attention.  The causal alignment with a
                              cached prefix is a reading (bottom-right), pinned only
                              by those invariants.
  * prefill_varlen_contiguous -- torch's float64 scaled-dot-product attention when
                              nothing is cached (causal and not), chunked equals
                              one-shot, and equal to prefill_varlen on the same keys
                              scattered into a shuffled paged pool.
  * merge_states           -- any split of the keys merges to the one-shot result.
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


# --------------------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns: a bf16 value is the upper 16 bits of a binary32."""
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return wide.view(np.float32).astype(np.float64)


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (``"bf16"`` as uint16 bits, ``"f32"`` as float32) -> float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------------------
# KV write through slot_mapping
# ("从零开始写Qwen3（六）PagedAttention", 自己来实现: the write kernel copies token n's
#  HIDDEN_DIM values to row slot_mapping[n] of the cache and returns early when the
#  slot is negative)
# --------------------------------------------------------------------------------------

def write_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
             v_new: np.ndarray, slot_mapping) -> tuple[np.ndarray, np.ndarray]:
    """Return copies of both pools with token n's K and V rows stored at its slot.

    Pools are ``[num_blocks, B, Hkv, d]``; viewed flat they are ``[num_blocks*B,
    Hkv*d]`` rows, and a slot is a row index of that view.  Negative slots are
    skipped.  The copy is bitwise: rows are moved as raw storage words.
    """
    nb, bs, hkv, d = k_pool.shape
    k_rows = k_pool.reshape(nb * bs, hkv * d).copy()
    v_rows = v_pool.reshape(nb * bs, hkv * d).copy()
    for n, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        if slot >= nb * bs:
            raise IndexError(f"slot {slot} outside a pool of {nb * bs} rows")
        k_rows[slot] = k_new[n].reshape(-1)
        v_rows[slot] = v_new[n].reshape(-1)
    return k_rows.reshape(k_pool.shape), v_rows.reshape(v_pool.shape)


def copy_blocks(k_pool: np.ndarray, v_pool: np.ndarray, src, dst):
    """Copy-on-write data step ("Paged attention 与 online softmax" §11.3): block
    dst[i] receives a bitwise copy of block src[i], in K and in V."""
    k = k_pool.copy()
    v = v_pool.copy()
    for s, t in zip(np.asarray(src).tolist(), np.asarray(dst).tolist()):
        k[t] = k_pool[s]
        v[t] = v_pool[s]
    return k, v


# --------------------------------------------------------------------------------------
# logical -> physical translation ("Paged attention 与 online softmax" §11.1)
# --------------------------------------------------------------------------------------

def locate(table_row, p: int, block_size: int) -> tuple[int, int]:
    """Logical token p -> (physical block, slot within the block).

    The logical block is floor(p / B), the slot is p mod B, and the physical block
    is the table entry of the logical block.
    """
    logical_block = p // block_size
    slot = p % block_size
    return int(table_row[logical_block]), slot


def element_offset(phys: int, slot: int, block_size: int, kv_dim: int,
                   head: int = 0, head_dim: int = 0, e: int = 0) -> int:
    """Element offset of (phys, slot, head, e) in one pool.

    §11.1 gives the start of the token's vector as phys*B*kvDim + slot*kvDim; the
    head and element offsets inside the kvDim-long row follow the row-major
    ``[Hkv, d]`` order of the cache row.
    """
    return phys * block_size * kv_dim + slot * kv_dim + head * head_dim + e


def gather(pool: np.ndarray, table_row, n_keys: int) -> tuple[np.ndarray, np.ndarray]:
    """Stage A of §11.2: copy the first n_keys logical tokens of one sequence out of
    the paged pool into a contiguous ``[n, Hkv, d]`` array.

    Returns ``(rows, positions)``: the positions are the logical indices that were
    gathered.  A key whose block-table entry is negative (an unassigned block) is
    left out, so it takes no part in the softmax.
    """
    block_size = pool.shape[1]
    positions = np.arange(n_keys, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[positions // block_size]
    slot = positions % block_size
    keep = phys >= 0
    return pool[phys[keep], slot[keep]], positions[keep]


# --------------------------------------------------------------------------------------
# softmax attention, two-pass (the plain definition)
# --------------------------------------------------------------------------------------

def attend(q_row: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query row, in two passes (max, then sum).

    An empty key set gives a zero vector (no key visible).
    """
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1], dtype=np.float64)
    s = scale * (keys @ q_row)
    m = s.max()
    p = np.exp(s - m)
    return (p @ values) / p.sum()


def decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_table,
           seqlens_k, scale: float, dtype: str) -> np.ndarray:
    """One query token per sequence against its paged cache.

    Follows the decode path of "Sayfalı dikkat" (Çözme yolu) and the
    ``flash_attn_with_kvcache`` call of "从零开始写Qwen3（六）": sequence b attends to
    its first seqlens_k[b] cached keys, read through row b of block_table.  With
    Hq query heads and Hkv KV heads, query head h uses KV head floor(h / (Hq/Hkv)).
    The single query sits at the last position, so a causal mask removes nothing.

    q: ``[batch, Hq, d]``; pools ``[num_blocks, B, Hkv, d]``; returns float64
    ``[batch, Hq, d]``.
    """
    batch, hq, d = q.shape
    hkv = k_pool.shape[2]
    group = hq // hkv
    qf = to_f64(q, dtype)
    table = np.asarray(block_table)
    out = np.zeros((batch, hq, d), dtype=np.float64)
    for b in range(batch):
        k_rows, _ = gather(k_pool, table[b], int(seqlens_k[b]))
        v_rows, _ = gather(v_pool, table[b], int(seqlens_k[b]))
        kf = to_f64(k_rows, dtype)
        vf = to_f64(v_rows, dtype)
        for h in range(hq):
            out[b, h] = attend(qf[b, h], kf[:, h // group], vf[:, h // group], scale)
    return out


def prefill_varlen(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, cu_seqlens_q,
                   cu_seqlens_k, block_table, scale: float, causal: bool,
                   dtype: str) -> np.ndarray:
    """Packed (varlen) prefill whose keys are read through the block table.

    Request i owns query rows [cu_q[i], cu_q[i+1]) of the packed ``[sum_q, Hq, d]``
    q ("Sayfalı dikkat", Değişken uzunluklu yol; "从零开始写Qwen3（六）", packed 模式).
    Its key count is k_len = cu_k[i+1] - cu_k[i]; with a block table the keys come
    from the paged cache, so only these differences are used (fast-attn 库的使用,
    "一个小细节").  When causal, query row t of the request is the token at logical
    position c + t with c = k_len - q_len cached tokens before it, and it sees keys
    j <= c + t (bottom-right alignment; the pages fix only ``causal=True``).
    A row that sees no key outputs zeros.
    """
    total_q, hq, d = q.shape
    hkv = k_pool.shape[2]
    group = hq // hkv
    qf = to_f64(q, dtype)
    table = np.asarray(block_table)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    out = np.zeros((total_q, hq, d), dtype=np.float64)
    for i in range(len(cu_q) - 1):
        q_len = int(cu_q[i + 1] - cu_q[i])
        k_len = int(cu_k[i + 1] - cu_k[i])
        cached = k_len - q_len
        k_rows, pos = gather(k_pool, table[i], k_len)
        v_rows, _ = gather(v_pool, table[i], k_len)
        kf = to_f64(k_rows, dtype)
        vf = to_f64(v_rows, dtype)
        for t in range(q_len):
            # gathered positions ascend, so the keys a row may see form a prefix
            n_visible = int(np.searchsorted(pos, cached + t, side="right")) if causal else len(pos)
            row = int(cu_q[i]) + t
            for h in range(hq):
                out[row, h] = attend(qf[row, h], kf[:n_visible, h // group],
                                     vf[:n_visible, h // group], scale)
    return out


def prefill_varlen_contiguous(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens_q,
                              cu_seqlens_k, scale: float, causal: bool, dtype: str) -> np.ndarray:
    """Packed (varlen) prefill with contiguous keys: the same call without a block
    table ("从零开始写Qwen3（六）", fast-attn 库的使用; "Sayfalı dikkat", Değişken uzunluklu
    yol), so k and v are packed like q, ``[sum_k, Hkv, d]``, and request i's keys are
    rows [cu_k[i], cu_k[i+1]).  Visibility as in prefill_varlen: with c = k_len - q_len,
    query row t sees keys j <= c + t when causal, all keys otherwise; no key -> zeros.
    """
    total_q, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    qf, kf, vf = to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype)
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    out = np.zeros((total_q, hq, d), dtype=np.float64)
    for i in range(len(cu_q) - 1):
        q_len = int(cu_q[i + 1] - cu_q[i])
        k0, k_len = int(cu_k[i]), int(cu_k[i + 1] - cu_k[i])
        cached = k_len - q_len
        for t in range(q_len):
            n_visible = min(max(cached + t + 1, 0), k_len) if causal else k_len
            row = int(cu_q[i]) + t
            keys = kf[k0:k0 + n_visible]
            vals = vf[k0:k0 + n_visible]
            for h in range(hq):
                out[row, h] = attend(qf[row, h], keys[:, h // group], vals[:, h // group], scale)
    return out


def dense_attention(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray,
                    scale: float, mask: np.ndarray | None = None) -> np.ndarray:
    """Textbook attention softmax(scale * Q K^T [masked]) V on contiguous float64
    arrays, row by row; used as the brute-force cross-check of the paged oracle."""
    out = np.zeros((q_rows.shape[0], values.shape[-1]), dtype=np.float64)
    for r in range(q_rows.shape[0]):
        keep = np.ones(keys.shape[0], dtype=bool) if mask is None else mask[r]
        if not keep.any():
            continue
        s = scale * np.array([float(np.dot(q_rows[r], keys[j])) for j in range(keys.shape[0])])
        w = np.where(keep, np.exp(s - s[keep].max()), 0.0)
        out[r] = (w / w.sum()) @ values
    return out


# --------------------------------------------------------------------------------------
# online softmax (题目2) and the block merge (§11.2)
# --------------------------------------------------------------------------------------

def online_softmax_trace(xs) -> list[tuple[float, float]]:
    """Scalar online softmax of 题目2: start from [m, l] = [-inf, 0]; on each new x,
    m' = max(m, x) and l' = l * e^(m - m') + e^(x - m').  Returns every (m, l)."""
    m, l = NEG_INF, 0.0
    trace = []
    for x in xs:
        m_new = max(m, float(x))
        l = l * math.exp(m - m_new) + math.exp(float(x) - m_new)
        m = m_new
        trace.append((m, l))
    return trace


def block_state(scores: np.ndarray, values: np.ndarray):
    """Statistics of one block of keys (§11.2): block max m_b, l_b = sum e^(s - m_b)
    and o_b = sum e^(s - m_b) v.  An empty block is (-inf, 0, 0)."""
    d = values.shape[-1]
    if scores.shape[0] == 0:
        return NEG_INF, 0.0, np.zeros(d, dtype=np.float64)
    m_b = float(scores.max())
    w = np.exp(scores - m_b)
    return m_b, float(w.sum()), w @ values


def merge_states(state, block):
    """The boxed merge of §11.2: m_new = max(m, m_b); both accumulators are rescaled
    by e^(m - m_new) and e^(m_b - m_new) and added.  When both maxima are -inf
    (nothing seen yet) the state stays (-inf, 0, 0)."""
    m, l, o = state
    m_b, l_b, o_b = block
    m_new = max(m, m_b)
    if m_new == NEG_INF:
        return NEG_INF, 0.0, np.zeros_like(o)
    a = math.exp(m - m_new)
    b = math.exp(m_b - m_new)
    return m_new, l * a + l_b * b, o * a + o_b * b


def blockwise_attend(q_row: np.ndarray, keys: np.ndarray, values: np.ndarray,
                     scale: float, boundaries) -> np.ndarray:
    """Stage B of §11.2: fold the keys block by block with merge_states and return
    o / l.  ``boundaries`` are the split points (any split gives the same result up
    to rounding, which is what §11.2 proves)."""
    s = scale * (keys @ q_row)
    cuts = [0] + [int(c) for c in boundaries] + [keys.shape[0]]
    state = (NEG_INF, 0.0, np.zeros(values.shape[-1], dtype=np.float64))
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        state = merge_states(state, block_state(s[lo:hi], values[lo:hi]))
    m, l, o = state
    return o / l if l > 0 else np.zeros_like(o)


def flash_tiles(Q: np.ndarray, K: np.ndarray, V: np.ndarray, br: int, bc: int):
    """The simplified FlashAttention loop of 题目3: Q tiles outside, K/V tiles inside,
    per-row state O (unnormalised), m and l; scale 1/sqrt(d); normalise at the end.

    Returns ``(O, steps)`` where ``steps[i]`` lists, for Q tile i and every K/V tile,
    the dict ``{"m", "l", "correction"}`` after that tile (correction is the
    e^(m_old - m_new) factor applied to the old state).
    """
    n, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((n, V.shape[1]), dtype=np.float64)
    steps = []
    for r0 in range(0, n, br):
        Qi = Q[r0:r0 + br]
        O = np.zeros((Qi.shape[0], V.shape[1]))
        m = np.full(Qi.shape[0], NEG_INF)
        l = np.zeros(Qi.shape[0])
        tile_steps = []
        for c0 in range(0, K.shape[0], bc):
            S = (Qi @ K[c0:c0 + bc].T) * scale
            m_new = np.maximum(m, S.max(axis=1))
            corr = np.exp(m - m_new)
            P = np.exp(S - m_new[:, None])
            l = l * corr + P.sum(axis=1)
            O = O * corr[:, None] + P @ V[c0:c0 + bc]
            m = m_new
            tile_steps.append({"m": m.copy(), "l": l.copy(), "correction": corr.copy()})
        out[r0:r0 + br] = O / l[:, None]
        steps.append(tile_steps)
    return out, steps

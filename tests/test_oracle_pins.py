"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: values the
pages print (tests/golden/*.json, each with its citation), closed forms derived by
hand, torch's float64 scaled-dot-product attention as an independent library
routine, and invariants (any block split merges to the same result, relabelling
physical blocks changes nothing, chunked prefill equals one-shot prefill).
The mutation tests at the end plant plausible mistakes in the oracle and check that
one of these pins catches each of them.
"""

import math
import random

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import blocks as K


# --------------------------------------------------------------------------------------
# helpers: tiny paged problems built by hand (independent of the library and of the
# workload generator)
# --------------------------------------------------------------------------------------

def _paged_from_dense(dense_k, dense_v, block_size, num_blocks, rng):
    """Scatter per-sequence contiguous [n, Hkv, d] float64 arrays into NaN-filled
    pools with randomly chosen physical blocks; returns pools and the table."""
    hkv, d = dense_k[0].shape[1:]
    widths = [-(-len(k) // block_size) for k in dense_k]
    width = max(widths + [1])
    kp = np.full((num_blocks, block_size, hkv, d), np.nan)
    vp = np.full((num_blocks, block_size, hkv, d), np.nan)
    ids = rng.sample(range(num_blocks), sum(widths))
    table = np.full((len(dense_k), width), -1, dtype=np.int64)
    it = iter(ids)
    for b, (k, v) in enumerate(zip(dense_k, dense_v)):
        for lb in range(widths[b]):
            table[b, lb] = next(it)
        for p in range(len(k)):
            kp[table[b, p // block_size], p % block_size] = k[p]
            vp[table[b, p // block_size], p % block_size] = v[p]
    return kp.astype(np.float32), vp.astype(np.float32), table


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _sdpa(q, k, v, scale, causal=False, group=1):
    """torch float64 SDPA on [n, H, d] arrays (heads first inside)."""
    qt = torch.tensor(q).permute(1, 0, 2)
    kt = torch.tensor(k).permute(1, 0, 2).repeat_interleave(group, dim=0)
    vt = torch.tensor(v).permute(1, 0, 2).repeat_interleave(group, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale, is_causal=causal)
    return o.permute(1, 0, 2).numpy()


# --------------------------------------------------------------------------------------
# 题目2 online softmax, §11.2 merge, 题目3 FlashAttention example
# --------------------------------------------------------------------------------------

def check_online_softmax(g):
    trace = A.online_softmax_trace(g["x"])
    for (m, l), (pm, pl) in zip(trace, g["printed_trace"]):
        assert m == pm
        assert abs(l - pl) <= g["printed_tolerance"]
    closed = sum(math.exp(x - max(g["x"])) for x in g["x"])
    assert abs(trace[-1][1] - closed) < 1e-9
    assert abs(trace[-1][1] - 1.5530018) < 1e-7


def test_online_softmax_trace(golden):
    check_online_softmax(golden("online_softmax_trace.json"))


def test_online_softmax_order_free():
    # the sum the trace reaches does not depend on the order of the elements
    xs = [0.3, -2.0, 5.5, 1.25, 5.5, -7.0]
    ref = sum(math.exp(x - max(xs)) for x in xs)
    for perm in ([5, 4, 3, 2, 1, 0], [2, 0, 4, 1, 5, 3]):
        assert abs(A.online_softmax_trace([xs[i] for i in perm])[-1][1] - ref) < 1e-12


def check_flash_example(g):
    Q, Kt, V = (np.array(g[n], dtype=np.float64) for n in ("Q", "K", "V"))
    out, steps = A.flash_tiles(Q, Kt, V, g["br"], g["bc"])
    q1 = steps[0]
    tol = g["printed_tolerance"]
    assert np.allclose(q1[0]["m"], g["printed_after_K1"]["m"], atol=tol)
    assert np.allclose(q1[0]["l"], g["printed_after_K1"]["l"], atol=tol)
    assert np.allclose(q1[0]["correction"], g["printed_correction"]["K1"], atol=tol)
    assert np.allclose(q1[1]["correction"], g["printed_correction"]["K2"], atol=tol)
    assert np.allclose(q1[1]["l"], g["derived_l_final_Q1"], atol=g["derived_tolerance"])
    assert np.allclose(out[:2], g["derived_O1"], atol=g["derived_tolerance"])
    # the whole output equals dense attention (the tiling changes nothing)
    assert np.allclose(out, _sdpa(Q[:, None], Kt[:, None], V[:, None], 1 / math.sqrt(2))[:, 0],
                       atol=1e-12)


def test_flash_attention_worked_example(golden):
    check_flash_example(golden("flash_tile_example.json"))


def check_merge_identity(seed=0):
    rng = np.random.default_rng(seed)
    n, d = 37, 16
    q = rng.normal(size=d)
    keys = rng.normal(size=(n, d)) * 3.0
    vals = rng.normal(size=(n, d))
    ref = _sdpa(q[None, None], keys[:, None], vals[:, None], 0.25)[0, 0]
    assert np.allclose(A.attend(q, keys, vals, 0.25), ref, atol=1e-12)
    for cuts in ([], [1], [16], [5, 6, 30], list(range(1, n)), [0, 0, 10, 10, 37]):
        got = A.blockwise_attend(q, keys, vals, 0.25, cuts)
        assert np.allclose(got, ref, atol=1e-12), cuts


def test_block_merge_identity():
    check_merge_identity()


def test_merge_of_empty_states_stays_empty():
    empty = (A.NEG_INF, 0.0, np.zeros(3))
    m, l, o = A.merge_states(empty, empty)
    assert m == A.NEG_INF and l == 0.0 and not np.any(o)
    blk = A.block_state(np.array([0.5, 1.5]), np.eye(2, 3))
    m, l, o = A.merge_states(empty, blk)
    assert (m, l) == (blk[0], blk[1]) and np.array_equal(o, blk[2])


# --------------------------------------------------------------------------------------
# §11.1 indexing, 题目5, the decode example of Sayfalı dikkat
# --------------------------------------------------------------------------------------

def check_block_table_example(g):
    B, table = g["block_size"], g["table"]
    layout = {}
    for p in range(len(table) * B):
        phys, off = A.locate(table, p, B)
        layout.setdefault(str(phys), []).append(p)
        assert off == p % B
    assert layout == g["printed_layout"]
    phys, off = A.locate(table, 9, B)
    t9 = g["printed_token9"]
    assert (9 // B, phys, off) == (t9["logical_block"], t9["physical_block"], t9["offset"])
    last = g["printed_ten_tokens_last_block"]
    in_last = [p for p in range(10) if A.locate(table, p, B)[0] == last["physical_block"]]
    assert in_last == last["tokens"] and (len(in_last) == B) == last["full"]
    assert K.slot_mapping([table], B, [0], [9]) == [5 * 4 + 1]


def test_block_table_example(golden):
    check_block_table_example(golden("block_table_example.json"))


def test_element_offset_matches_section_11_1():
    # §11.1: the K vector of (phys, slot) starts at phys*B*kvDim + slot*kvDim; times 4 bytes for fp32
    B, kv = 16, 1024
    assert A.element_offset(3, 5, B, kv) == 3 * 16 * 1024 + 5 * 1024
    pool = np.arange(8 * B * 2 * 4, dtype=np.float32).reshape(8, B, 2, 4)
    for phys, slot, h, e in [(0, 0, 0, 0), (7, 15, 1, 3), (3, 5, 1, 2)]:
        assert pool.reshape(-1)[A.element_offset(phys, slot, B, 8, h, 4, e)] == pool[phys, slot, h, e]


def check_decode_table_example(g):
    B = g["block_size"]
    table = g["printed_block_table"]
    lens = g["cache_seqlens"]
    slots = K.slot_mapping(table, B, range(len(lens)), lens)
    assert slots == g["derived_new_token_slots"]
    fits = [K.blocks_per_layer(n + 1, B) == K.blocks_per_layer(n, B) for n in lens]
    assert fits == g["printed_new_token_fits_existing_blocks"]
    assert [K.blocks_per_layer(n + 1, B) for n in lens] == g["printed_blocks_after_append"]
    assert [sum(1 for x in row if x >= 0) for row in table] == g["printed_blocks_after_append"]
    # replaying the example through the block manager reaches the printed table
    bm = K.BlockManager(8, initial_order=[2, 0, 1, 3, 5, 6, 4, 7])
    rows = []
    for n in lens:
        row = [-1] * 4
        bm.prepare_write(row, 0, n + 1, B)
        rows.append(row)
    assert rows == table


def test_decode_table_example(golden):
    check_decode_table_example(golden("decode_table_example.json"))


# --------------------------------------------------------------------------------------
# KV write
# --------------------------------------------------------------------------------------

def test_write_kv_bitwise_and_negative_slots():
    rng = random.Random(3)
    nb, B, hkv, d = 6, 4, 2, 8
    bits = np.random.default_rng(3).integers(0, 1 << 16, size=(nb, B, hkv, d), dtype=np.uint16)
    kp, vp = bits.copy(), bits[::-1].copy()
    k_new = np.random.default_rng(4).integers(0, 1 << 16, size=(5, hkv, d), dtype=np.uint16)
    v_new = k_new ^ np.uint16(0x5555)
    slots = [7, -1, 23, 0, -5]
    k2, v2 = A.write_kv(kp, vp, k_new, v_new, slots)
    flat_k, flat_v = k2.reshape(nb * B, -1), v2.reshape(nb * B, -1)
    for n, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(flat_k[s], k_new[n].reshape(-1))
            assert np.array_equal(flat_v[s], v_new[n].reshape(-1))
    untouched = [r for r in range(nb * B) if r not in (7, 23, 0)]
    assert np.array_equal(flat_k[untouched], kp.reshape(nb * B, -1)[untouched])
    # the row written at slot s is the one §11.1's offset formula addresses
    s = 23
    assert np.array_equal(k2.reshape(-1)[A.element_offset(s // B, s % B, B, hkv * d):][:hkv * d],
                          k_new[2].reshape(-1))
    # nan payloads survive bit for bit in float32 storage
    f = np.full((2, 2, 1, 2), np.nan, dtype=np.float32)
    payload = np.array([[[0x7FC00001, 0xFFC12345]]], dtype=np.uint32).view(np.float32)
    kf, _ = A.write_kv(f, f, payload, payload, [3])
    assert kf.reshape(4, 2)[3].view(np.uint32).tolist() == [0x7FC00001, 0xFFC12345]
    del rng


def _coded_pool(tag, nb, B, hkv, d, dtype):
    """A pool whose every element names itself: (tag, block, slot, head, dim) packed into
    the storage word, so any block read from the wrong place, or not copied, shows.  In
    float32 the codes are NaN payloads (quiet NaN, sign from the tag)."""
    idx = np.arange(nb * B * hkv * d, dtype=np.uint32).reshape(nb, B, hkv, d)
    if dtype == "bf16":
        return ((idx & np.uint32(0x3FFF)) | np.uint32(tag << 14)).astype(np.uint16)
    return (np.uint32(0x7FC00000 | (tag << 31)) | idx).view(np.float32)


def check_copy_blocks():
    """Copy-on-write data step ("Paged attention 与 online softmax" §11.3): before a shared
    block is written, a new block receives its contents; the old block is left as it was.
    Expected pools are built from the element codes directly (block s's codes moved to
    block t), not by any copying routine."""
    nb, B, hkv, d = 7, 2, 2, 4
    for dtype in ("bf16", "f32"):
        kp, vp = _coded_pool(0, nb, B, hkv, d, dtype), _coded_pool(1, nb, B, hkv, d, dtype)
        k_before, v_before = kp.copy(), vp.copy()
        pairs = [(4, 1), (0, 5), (6, 2)]
        k2, v2 = A.copy_blocks(kp, vp, [s for s, _ in pairs], [t for _, t in pairs])
        # the inputs are not modified
        assert kp.tobytes() == k_before.tobytes() and vp.tobytes() == v_before.tobytes()
        for tag, got in ((0, k2), (1, v2)):
            want = _coded_pool(tag, nb, B, hkv, d, dtype)
            for s, t in pairs:
                want[t] = _coded_pool(tag, nb, B, hkv, d, dtype)[s]
            assert got.dtype == want.dtype and got.shape == want.shape
            assert got.tobytes() == want.tobytes(), f"{dtype} pool {tag}: copied blocks differ"
        # an empty pair list changes nothing
        k3, v3 = A.copy_blocks(kp, vp, [], [])
        assert k3.tobytes() == kp.tobytes() and v3.tobytes() == vp.tobytes()


def test_copy_blocks_bitwise():
    check_copy_blocks()


def test_bf16_codec():
    pats = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049, 0x3EAA], dtype=np.uint16)
    got = A.bf16_bits_to_f64(pats)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == math.inf and got[3] == -math.inf
    assert got[4] == 2.0 ** -133 and got[5] == 0.0 and math.copysign(1, got[5]) == -1
    ref = torch.tensor(pats.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = A.bf16_bits_to_f64(allbits)
    theirs = torch.tensor(allbits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(theirs)
    assert np.array_equal(mine[finite], theirs[finite])
    assert np.array_equal(np.isnan(mine), np.isnan(theirs))


# --------------------------------------------------------------------------------------
# decode: brute force, special cases, invariants
# --------------------------------------------------------------------------------------

def _random_decode(seed, lens, hq, hkv, d, B, nb):
    rng = random.Random(seed)
    npr = np.random.default_rng(seed)
    dk = [_f32(npr.normal(size=(n, hkv, d))) for n in lens]
    dv = [_f32(npr.normal(size=(n, hkv, d))) for n in lens]
    kp, vp, table = _paged_from_dense(dk, dv, B, nb, rng)
    q = npr.normal(size=(len(lens), hq, d)).astype(np.float32)
    return q, kp, vp, table, dk, dv


def check_decode_brute_force(seed=1):
    lens = [1, 5, 17, 33]
    hq, hkv, d, B = 4, 2, 8, 4
    q, kp, vp, table, dk, dv = _random_decode(seed, lens, hq, hkv, d, B, 40)
    scale = 0.3
    out = A.decode(q, kp, vp, table, lens, scale, "f32")
    for b, n in enumerate(lens):
        ref = _sdpa(_f32(q[b])[None], dk[b], dv[b], scale, group=hq // hkv)[0]
        assert np.allclose(out[b], ref, atol=1e-12), b
        for h in range(hq):
            kb = dk[b][:, h // 2]
            brute = A.dense_attention(_f32(q[b, h])[None], kb, dv[b][:, h // 2], scale)[0]
            assert np.allclose(out[b, h], brute, atol=1e-12)


def test_decode_matches_dense_attention():
    check_decode_brute_force()


def test_decode_special_cases():
    hq, hkv, d, B = 2, 2, 8, 4
    q, kp, vp, table, dk, dv = _random_decode(5, [1, 9], hq, hkv, d, B, 8)
    out = A.decode(q, kp, vp, table, [1, 9], 0.7, "f32")
    assert np.array_equal(out[0], dv[0][0])                       # one key: its value exactly
    zero_q = np.zeros_like(q)
    out0 = A.decode(zero_q, kp, vp, table, [1, 9], 0.7, "f32")
    assert np.allclose(out0[1], dv[1].mean(axis=0), atol=1e-12)   # equal scores: the mean
    # Hq == Hkv is per-head multi-head attention
    for h in range(hq):
        assert np.allclose(out[1, h], _sdpa(_f32(q[1, h])[None, None], dk[1][:, h:h + 1],
                                            dv[1][:, h:h + 1], 0.7)[0, 0], atol=1e-12)
    # zero keys: zeros
    assert not np.any(A.decode(q, kp, vp, table, [0, 0], 0.7, "f32"))


def test_decode_relabelling_invariance():
    q, kp, vp, table, _, _ = _random_decode(7, [13, 3, 22], 4, 2, 8, 4, 30)
    out = A.decode(q, kp, vp, table, [13, 3, 22], 0.5, "f32")
    perm = np.random.default_rng(0).permutation(30)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    assert np.array_equal(A.decode(q, kp2, vp2, table2, [13, 3, 22], 0.5, "f32"), out)


def test_decode_bf16_decodes_storage():
    npr = np.random.default_rng(11)
    vals = torch.tensor(npr.normal(size=(2, 4, 2, 8)), dtype=torch.float32).to(torch.bfloat16)
    bits = vals.view(torch.int16).numpy().view(np.uint16)
    q = torch.tensor(npr.normal(size=(1, 2, 8)), dtype=torch.float32).to(torch.bfloat16)
    qbits = q.view(torch.int16).numpy().view(np.uint16)
    out = A.decode(qbits, bits, bits[::-1].copy(), [[1, 0]], [6], 0.4, "bf16")
    kf = vals.to(torch.float64).numpy()
    dense_k = np.concatenate([kf[1], kf[0]])[:6]
    dense_v = np.concatenate([kf[::-1][1], kf[::-1][0]])[:6]
    ref = _sdpa(q.to(torch.float64).numpy()[0][None], dense_k, dense_v, 0.4)[0]
    assert np.allclose(out[0], ref, atol=1e-12)


def test_unassigned_block_masks_its_keys():
    # a -1 entry inside the length: its keys take no part (never read)
    q, kp, vp, table, dk, dv = _random_decode(9, [12], 2, 1, 8, 4, 6)
    t = table.copy()
    t[0, 1] = -1
    out = A.decode(q, kp, vp, t, [12], 0.5, "f32")
    keep = [0, 1, 2, 3, 8, 9, 10, 11]
    ref = _sdpa(_f32(q[0])[None], dk[0][keep], dv[0][keep], 0.5, group=2)[0]
    assert np.allclose(out[0], ref, atol=1e-12)


# --------------------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------------------

def _random_prefill(seed, q_lens, k_lens, hq, hkv, d, B):
    rng = random.Random(seed)
    npr = np.random.default_rng(seed)
    dk = [_f32(npr.normal(size=(n, hkv, d))) for n in k_lens]
    dv = [_f32(npr.normal(size=(n, hkv, d))) for n in k_lens]
    kp, vp, table = _paged_from_dense(dk, dv, B, sum(-(-n // B) for n in k_lens) + 3, rng)
    q = npr.normal(size=(sum(q_lens), hq, d)).astype(np.float32)
    cu_q, _ = K.cu_seqlens(q_lens)
    cu_k, _ = K.cu_seqlens(k_lens)
    return q, kp, vp, table, cu_q, cu_k, dk, dv


def check_prefill_no_cache_is_causal_attention(seed=2):
    q_lens = [7, 1, 12]
    q, kp, vp, table, cu_q, cu_k, dk, dv = _random_prefill(seed, q_lens, q_lens, 4, 2, 8, 4)
    out = A.prefill_varlen(q, kp, vp, cu_q, cu_k, table, 0.35, True, "f32")
    for i, n in enumerate(q_lens):
        rows = slice(cu_q[i], cu_q[i + 1])
        ref = _sdpa(_f32(q[rows]), dk[i], dv[i], 0.35, causal=True, group=2)
        assert np.allclose(out[rows], ref, atol=1e-12)
    out_nc = A.prefill_varlen(q, kp, vp, cu_q, cu_k, table, 0.35, False, "f32")
    for i, n in enumerate(q_lens):
        rows = slice(cu_q[i], cu_q[i + 1])
        ref = _sdpa(_f32(q[rows]), dk[i], dv[i], 0.35, causal=False, group=2)
        assert np.allclose(out_nc[rows], ref, atol=1e-12)


def test_prefill_without_cache_is_causal_attention():
    check_prefill_no_cache_is_causal_attention()


def check_chunked_prefill_equals_one_shot(seed=4):
    # "分块预填充": a long prefill split into chunks, later chunks reading the cache,
    # must give every row the same output as the one-shot prefill.
    n, hq, hkv, d, B = 29, 4, 2, 8, 4
    q, kp, vp, table, cu_q, cu_k, _, _ = _random_prefill(seed, [n], [n], hq, hkv, d, B)
    full = A.prefill_varlen(q, kp, vp, cu_q, cu_k, table, 0.4, True, "f32")
    for cut in (1, 8, 13, 28):
        # chunk 2 only: q rows cut..n-1, key length n (cut of them cached)
        part = A.prefill_varlen(q[cut:], kp, vp, [0, n - cut], [0, n], table, 0.4, True, "f32")
        assert np.allclose(part, full[cut:], atol=1e-12), cut
    # the same two chunks packed as two requests of one batch
    two = np.concatenate([table, table])
    both = A.prefill_varlen(np.concatenate([q[:10], q[10:]]), kp, vp, [0, 10, n], [0, 10, 10 + n],
                            two, 0.4, True, "f32")
    assert np.allclose(both, full, atol=1e-12)


def test_chunked_prefill_equals_one_shot():
    check_chunked_prefill_equals_one_shot()


def test_prefill_single_query_equals_decode():
    q_lens, k_lens = [1, 1, 1], [5, 17, 9]
    q, kp, vp, table, cu_q, cu_k, _, _ = _random_prefill(6, q_lens, k_lens, 4, 2, 8, 4)
    pre = A.prefill_varlen(q, kp, vp, cu_q, cu_k, table, 0.5, True, "f32")
    dec = A.decode(q, kp, vp, table, k_lens, 0.5, "f32")
    assert np.allclose(pre, dec, atol=1e-13)


def test_prefill_rows_without_keys_are_zero(golden):
    # the varlen example's lengths: request 0 has 10 queries and no keys at all
    g = golden("varlen_example.json")
    q, kp, vp, table, _, _, _, _ = _random_prefill(8, [10, 3, 1], [1, 1, 7], 2, 1, 8, 4)
    out = A.prefill_varlen(q, kp, vp, g["printed_cu_seq_lens_q"], g["printed_cu_seq_lens_k"],
                           table, 0.5, True, "f32")
    assert not np.any(out[:10])                       # k_len 0
    assert not np.any(out[10:12]) and np.any(out[12])  # k_len 1, q_len 3: only the last row sees it
    assert np.any(out[13])


def _random_contiguous(seed, q_lens, k_lens, hq, hkv, d):
    npr = np.random.default_rng(seed)
    k = npr.normal(size=(sum(k_lens), hkv, d)).astype(np.float32)
    v = npr.normal(size=(sum(k_lens), hkv, d)).astype(np.float32)
    q = npr.normal(size=(sum(q_lens), hq, d)).astype(np.float32)
    return q, k, v, K.cu_seqlens(q_lens)[0], K.cu_seqlens(k_lens)[0]


def check_contiguous_prefill(seed=10):
    # nothing cached: torch's causal / full SDPA per request
    lens = [7, 1, 12, 0, 5]
    q, k, v, cu_q, cu_k = _random_contiguous(seed, lens, lens, 6, 3, 8)
    for causal in (True, False):
        out = A.prefill_varlen_contiguous(q, k, v, cu_q, cu_k, 0.3, causal, "f32")
        for i in range(len(lens)):
            if not lens[i]:
                continue
            rq, rk = slice(cu_q[i], cu_q[i + 1]), slice(cu_k[i], cu_k[i + 1])
            ref = _sdpa(_f32(q[rq]), _f32(k[rk]), _f32(v[rk]), 0.3, causal=causal, group=2)
            assert np.allclose(out[rq], ref, atol=1e-12), (i, causal)
    # a cached prefix (k_len > q_len): the last rows of the one-shot causal prefill
    n = 23
    q, k, v, _, _ = _random_contiguous(seed + 1, [n], [n], 4, 2, 8)
    full = A.prefill_varlen_contiguous(q, k, v, [0, n], [0, n], 0.5, True, "f32")
    for cut in (1, 9, 22):
        part = A.prefill_varlen_contiguous(q[cut:], k, v, [0, n - cut], [0, n], 0.5, True, "f32")
        assert np.allclose(part, full[cut:], atol=1e-12), cut
    # packed behind another request: the same rows
    k2 = np.concatenate([k[:4], k])
    v2 = np.concatenate([v[:4], v])
    both = A.prefill_varlen_contiguous(np.concatenate([q[:3], q[5:]]), k2, v2, [0, 3, 3 + n - 5],
                                       [0, 4, 4 + n], 0.5, True, "f32")
    assert np.allclose(both[3:], full[5:], atol=1e-12)


def test_contiguous_prefill_pins():
    check_contiguous_prefill()


def test_contiguous_prefill_equals_paged_prefill():
    q_lens, k_lens = [5, 1, 17, 3], [9, 30, 17, 3]
    q, kp, vp, table, cu_q, cu_k, dk, dv = _random_prefill(12, q_lens, k_lens, 4, 2, 8, 4)
    k, v = np.concatenate(dk).astype(np.float32), np.concatenate(dv).astype(np.float32)
    for causal in (True, False):
        paged = A.prefill_varlen(q, kp, vp, cu_q, cu_k, table, 0.45, causal, "f32")
        contig = A.prefill_varlen_contiguous(q, k, v, cu_q, cu_k, 0.45, causal, "f32")
        assert np.array_equal(paged, contig)


# --------------------------------------------------------------------------------------
# block manager and sizing
# --------------------------------------------------------------------------------------

def check_prefix_refcount_example(g, Manager=K.BlockManager):
    B = g["block_size"]
    bm = Manager(16)
    base = [-1] * 3
    bm.prepare_write(base, 0, 4, B)
    assert base[:2] == g["printed_base"]["table"]
    assert {str(i): bm.refs[i] for i in base[:2]} == g["printed_base"]["refs"]
    r1 = bm.share(base)
    bm.prepare_write(r1, 4, 2, B)
    assert r1 == g["printed_after_request1"]["table"]
    assert {str(i): bm.refs[i] for i in r1} == g["printed_after_request1"]["refs"]
    r2 = bm.share(base)
    bm.prepare_write(r2, 4, 2, B)
    assert r2 == g["printed_after_request2"]["table"]
    assert {str(i): bm.refs[i] for i in r2} == g["printed_after_request2"]["refs"]
    free_before = bm.num_free()
    bm.release_table(r1)
    freed = bm.num_free() - free_before
    assert freed == len(g["printed_after_request1_ends"]["freed"])
    assert bm.free[-1] == g["printed_after_request1_ends"]["freed"][0]
    assert {str(i): bm.refs[i] for i in (0, 1, 3)} == g["printed_after_request1_ends"]["refs"]
    assert r2 == g["printed_request2_final_table"]
    assert 2 * B == g["printed_saving_tokens"]
    # the freed block is the next one handed out (it went back on top of the stack)
    assert bm.alloc(1) == [2]


def test_prefix_refcount_example(golden):
    check_prefix_refcount_example(golden("prefix_refcount_example.json"))


def test_fnv1a64_reference_vectors(golden):
    for text, hexval in golden("fnv1a64_vectors.json")["vectors"]:
        assert K.fnv1a64(text.encode()) == int(hexval, 16)
    # the chained block hash is FNV-1a over (previous hash LE64, token ids LE32)
    assert K.block_hash([], 0) == K.fnv1a64(bytes(8))
    assert K.block_hash([1, -1], 5) == K.fnv1a64((5).to_bytes(8, "little") + b"\x01\0\0\0" + b"\xff" * 4)


def check_prefix_cache_example(g, Manager=K.BlockManager):
    """题目6 from token ids: the hash lookup decides sharing, not explicit calls."""
    B = g["block_size"]
    A_, B_, C_, D_, E_, F_, G_, H_ = range(1, 9)
    bm = Manager(16)
    base, hits = bm.allocate_prefix([A_, B_, C_, D_], B, 3)
    assert base[:2] == g["printed_base"]["table"] and hits == 0
    assert {str(i): bm.refs[i] for i in base[:2]} == g["printed_base"]["refs"]
    r1, hits = bm.allocate_prefix([A_, B_, C_, D_, E_, F_], B, 3)
    assert r1 == g["printed_after_request1"]["table"] and hits == 2
    assert {str(i): bm.refs[i] for i in r1} == g["printed_after_request1"]["refs"]
    r2, hits = bm.allocate_prefix([A_, B_, C_, D_, G_, H_], B, 3)
    assert r2 == g["printed_after_request2"]["table"] and hits == 2
    assert {str(i): bm.refs[i] for i in r2} == g["printed_after_request2"]["refs"]
    bm.release_table(r1)
    assert {str(i): bm.refs[i] for i in (0, 1, 3)} == g["printed_after_request1_ends"]["refs"]
    assert bm.free[-1] == g["printed_after_request1_ends"]["freed"][0]
    # block 2 left the cache: [E, F] misses now and takes the freed block again
    r3, hits = bm.allocate_prefix([A_, B_, C_, D_, E_, F_], B, 3)
    assert r3 == [0, 1, 2] and hits == 2
    # the same tokens after a different prefix do not hit (the hash is chained)
    r4, hits = bm.allocate_prefix([G_, H_, E_, F_], B, 2)
    assert hits == 0 and r4[1] != 2


def test_prefix_cache_example(golden):
    check_prefix_cache_example(golden("prefix_refcount_example.json"))


def test_waste_and_growth(golden):
    g = golden("waste_example.json")
    alloc, waste = K.contiguous_waste(g["used"], g["max_len"])
    assert (alloc, waste) == (g["printed_contiguous"]["allocated"], g["printed_contiguous"]["wasted"])
    assert round(100 * waste / alloc, 2) == g["printed_contiguous"]["waste_pct"]
    alloc, waste = K.paged_waste(g["used"], g["block_size"])
    assert (alloc, waste) == (g["printed_paged"]["allocated"], g["printed_paged"]["wasted"])
    assert round(100 * waste / alloc, 2) == g["printed_paged"]["waste_pct"]
    bm = K.BlockManager(g["pool_blocks"])
    rows = []
    for u in g["used"]:
        row = [-1] * 3
        bm.prepare_write(row, 0, u, g["block_size"])
        rows.append(row)
    assert [sum(x >= 0 for x in r) for r in rows] == g["printed_paged"]["blocks"]
    free0 = bm.num_free()
    bm.prepare_write(rows[1], 5, 2, g["block_size"])       # B grows 5 -> 7
    assert free0 - bm.num_free() == g["printed_growth"]["5_to_7_new_blocks"]
    bm.prepare_write(rows[1], 7, 2, g["block_size"])       # ... -> 9
    assert free0 - bm.num_free() == g["printed_growth"]["5_to_9_new_blocks"]


def test_block_manager_errors_and_cow():
    bm = K.BlockManager(4, initial_order=[3, 1, 0, 2])
    assert bm.alloc(2) == [3, 1]
    with pytest.raises(K.OutOfBlocks):
        bm.alloc(3)
    assert bm.num_free() == 2                       # all or nothing
    with pytest.raises(K.RefcountError):
        bm.decref(0)
    row = [3, 1, -1]
    bm.incref(1)                                    # someone else holds block 1
    copies = bm.prepare_write(row, 5, 6, 4)         # touches logical blocks 1 and 2
    assert copies == [(1, 0)] and row == [3, 0, 2]
    assert bm.refs[1] == 1 and bm.refs[0] == 1 and bm.refs[2] == 1
    row2 = [3, 1, -1]
    bm.incref(3)
    bm.incref(1)
    with pytest.raises(K.OutOfBlocks):              # needs 3 blocks, none free
        bm.prepare_write(row2, 0, 12, 4)
    assert row2 == [3, 1, -1] and bm.refs[3] == 2


def test_pool_size_example(golden):
    g = golden("pool_size_example.json")
    B, T, L, kv = g["block_size"], g["tokens"], g["layers"], g["kv_dim"]
    assert K.blocks_per_layer(T, B) == g["printed_blocks_per_layer"]
    n = K.total_blocks(T, B, L)
    assert n == g["printed_total_blocks"]
    assert K.block_bytes(B, kv, g["elem_bytes"]) == g["printed_block_bytes"]
    total = K.pool_bytes(n, B, kv, g["elem_bytes"])
    assert total == 25_690_112 and abs(total / 2**20 - g["printed_total_mib_approx"]) < 0.05
    assert K.last_block_fill(T, B) == g["printed_last_block_slots"]
    assert max(K.blocks_per_layer(t, B) * B - t for t in range(1, 200)) == g["printed_max_internal_waste_tokens_per_layer"]


def test_kv_size_example(golden):
    g = golden("kv_size_example.json")
    per = K.kv_bytes_per_token(g["layers"], g["kv_dim"], g["elem_bytes"])
    assert per == g["printed_bytes_per_token_kib"] * 1024
    assert per * g["tokens"] == g["printed_total_mib"] * 2**20
    assert abs(per * g["tokens"] / 2**30 - g["printed_total_gib_approx"]) < 0.05


def test_varlen_metadata_example(golden):
    g = golden("varlen_example.json")
    cu_q, max_q = K.cu_seqlens(g["q_lengths"])
    cu_k, max_k = K.cu_seqlens(g["k_lengths"])
    assert cu_q == g["printed_cu_seq_lens_q"] and cu_k == g["printed_cu_seq_lens_k"]
    assert (max_q, max_k) == (g["printed_max_length_q"], g["printed_max_length_k"])
    assert K.request_index(cu_q) == g["printed_q_request_index"]
    assert K.request_index(cu_k) == g["printed_k_request_index"]


# --------------------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# --------------------------------------------------------------------------------------

def _caught(monkeypatch, target, attr, wrong, check):
    with monkeypatch.context() as m:
        m.setattr(target, attr, wrong)
        with pytest.raises(AssertionError):
            check()


def test_planted_mistakes_are_caught(monkeypatch, golden):
    orig_locate = A.locate
    orig_merge = A.merge_states
    orig_gather = A.gather
    orig_attend = A.attend

    # offset taken from the wrong end of the block
    _caught(monkeypatch, A, "locate",
            lambda row, p, B: (int(row[p // B]), B - 1 - p % B),
            lambda: check_block_table_example(golden("block_table_example.json")))
    # merge forgets to rescale the old accumulator
    def bad_merge(state, block):
        m, l, o = state
        m_b, l_b, o_b = block
        m_new = max(m, m_b)
        if m_new == A.NEG_INF:
            return orig_merge(state, block)
        b = math.exp(m_b - m_new)
        return m_new, l + l_b * b, o + o_b * b
    _caught(monkeypatch, A, "merge_states", bad_merge, check_merge_identity)
    # gather reads slot p // B instead of p mod B
    def bad_gather(pool, row, n):
        pos = np.arange(n)
        phys = np.asarray(row)[pos // pool.shape[1]]
        return pool[phys, (pos // pool.shape[1]) % pool.shape[1]], pos
    _caught(monkeypatch, A, "gather", bad_gather, check_decode_brute_force)
    # softmax sign flipped
    _caught(monkeypatch, A, "attend",
            lambda q, k, v, s: orig_attend(q, k, v, -s), check_decode_brute_force)
    # causal mask aligned top-left instead of after the cached prefix
    def top_left(q, kp, vp, cu_q, cu_k, table, scale, causal, dtype):
        out = np.zeros((q.shape[0],) + q.shape[1:], dtype=np.float64)
        for i in range(len(cu_q) - 1):
            for t in range(cu_q[i + 1] - cu_q[i]):
                kk, _ = orig_gather(kp, table[i], t + 1)
                vv, _ = orig_gather(vp, table[i], t + 1)
                for h in range(q.shape[1]):
                    g = q.shape[1] // kp.shape[2]
                    out[cu_q[i] + t, h] = orig_attend(_f32(q[cu_q[i] + t, h]), _f32(kk[:, h // g]),
                                                      _f32(vv[:, h // g]), scale)
        return out
    _caught(monkeypatch, A, "prefill_varlen", top_left, check_chunked_prefill_equals_one_shot)
    # contiguous prefill: (a) keys sliced at the query offsets, (b) causal limit off by
    # one (a row does not see its own key)
    def contiguous_variant(start, visible):
        def run(q, k, v, cu_q, cu_k, scale, causal, dtype):
            out = np.zeros(q.shape, dtype=np.float64)
            g = q.shape[1] // k.shape[1]
            for i in range(len(cu_q) - 1):
                ql, kl = cu_q[i + 1] - cu_q[i], cu_k[i + 1] - cu_k[i]
                k0 = start(cu_q, cu_k, i)
                for t in range(ql):
                    nv = visible(ql, kl, t) if causal else kl
                    for h in range(q.shape[1]):
                        out[cu_q[i] + t, h] = orig_attend(
                            _f32(q[cu_q[i] + t, h]), _f32(k[k0:k0 + nv, h // g]),
                            _f32(v[k0:k0 + nv, h // g]), scale)
            return out
        return run
    good_visible = lambda ql, kl, t: min(max(kl - ql + t + 1, 0), kl)
    _caught(monkeypatch, A, "prefill_varlen_contiguous",
            contiguous_variant(lambda cq, ck, i: cq[i], good_visible), check_contiguous_prefill)
    _caught(monkeypatch, A, "prefill_varlen_contiguous",
            contiguous_variant(lambda cq, ck, i: ck[i], lambda ql, kl, t: min(max(kl - ql + t, 0), kl)),
            check_contiguous_prefill)
    # (the correct variant passes, so the two above fail for their mistake alone)
    with monkeypatch.context() as m:
        m.setattr(A, "prefill_varlen_contiguous",
                  contiguous_variant(lambda cq, ck, i: ck[i], good_visible))
        check_contiguous_prefill()
    # copy-on-write: (a) source and destination swapped, (b) only the K pool copied
    orig_copy = A.copy_blocks
    _caught(monkeypatch, A, "copy_blocks",
            lambda k, v, src, dst: orig_copy(k, v, dst, src), check_copy_blocks)
    _caught(monkeypatch, A, "copy_blocks",
            lambda k, v, src, dst: (orig_copy(k, v, src, dst)[0], v.copy()), check_copy_blocks)
    # the freed block is appended at the bottom of the free stack
    # the prefix hash ignores the chaining
    with monkeypatch.context() as m:
        m.setattr(K, "block_hash", lambda tokens, prefix: K.fnv1a64(b"".join(
            int(t).to_bytes(4, "little", signed=True) for t in tokens)))
        with pytest.raises(AssertionError):
            check_prefix_cache_example(golden("prefix_refcount_example.json"))

    class BottomFree(K.BlockManager):
        def decref(self, block):
            self.refs[block] -= 1
            if self.refs[block] == 0:
                self.free.insert(0, block)
    with pytest.raises(AssertionError):
        check_prefix_refcount_example(golden("prefix_refcount_example.json"), BottomFree)
    del orig_locate

"""Oracle for the host side: block manager, block tables, slot mapping, packed-batch
metadata and pool sizing.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pure Python.

Pins (tests/test_oracle_pins.py):
  * BlockManager            -- 题目6 reference-count trace, 题目4 growth examples.
  * slot_mapping            -- 题目5 (token 9 -> block 5, offset 1) and the
                               Sayfalı dikkat decode example.
  * cu_seqlens              -- Sayfalı dikkat varlen example ([10,3,1] / [0,1,7]).
  * pool sizing / waste     -- §11.1 example (196 blocks, 128 KiB, ~24.5 MiB),
                               KVCache大小计算 (112 KiB per token, 4480 MiB),
                               题目4 waste (58.33 % versus 37.5 %).
"""

from __future__ import annotations


FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


class OutOfBlocks(RuntimeError):
    pass


class RefcountError(RuntimeError):
    pass


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


# --------------------------------------------------------------------------------------
# block manager ("Paged attention 与 online softmax" §11.3; 题目4 and 题目6)
# --------------------------------------------------------------------------------------

class BlockManager:
    """Reference-counted pool of physical block ids with a free stack.

    §11.3: refs[p] counts the block tables (or prefix-cache holders) that point at
    block p; allocation sets it to 1, sharing adds 1, releasing subtracts 1, and only
    a count that reaches 0 puts the block back on the free stack.  题目6 hands out
    free blocks in the order 0, 1, 2, ...; a released block goes back on top of the
    stack, so it is the next one handed out.  ``initial_order`` replaces 0, 1, 2, ...
    by any permutation (the first entry is handed out first).
    """

    def __init__(self, num_blocks: int, initial_order=None):
        order = list(range(num_blocks)) if initial_order is None else [int(x) for x in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("initial_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.refs = [0] * num_blocks
        self.free = list(reversed(order))  # the top of the stack is the end of the list
        # prefix cache (题目6): hash_to_block_id and, per registered block, its hash and
        # the token ids it holds (checked on a hit)
        self.hash_to_block = {}
        self.block_hash = {}
        self.block_tokens = {}

    def num_free(self) -> int:
        return len(self.free)

    def alloc(self, n: int) -> list[int]:
        """Take n blocks (all or nothing), each with refs = 1."""
        if n > len(self.free):
            raise OutOfBlocks(f"need {n} blocks, {len(self.free)} free")
        ids = [self.free.pop() for _ in range(n)]
        for i in ids:
            self.refs[i] = 1
        return ids

    def incref(self, block: int) -> None:
        if self.refs[block] <= 0:
            raise RefcountError(f"block {block} is not allocated")
        self.refs[block] += 1

    def decref(self, block: int) -> None:
        if self.refs[block] <= 0:
            raise RefcountError(f"block {block} is not allocated")
        self.refs[block] -= 1
        if self.refs[block] == 0:
            self._forget(block)        # a freed block leaves hash_to_block_id (题目6, step 4)
            self.free.append(block)

    def _forget(self, block: int) -> None:
        h = self.block_hash.pop(block, None)
        if h is not None:
            del self.hash_to_block[h]
            del self.block_tokens[block]

    def allocate_prefix(self, tokens, block_size: int, width: int):
        """Table row for a request's token ids, sharing cached full blocks (题目6).

        Full block i gets the chained hash h_i = block_hash(tokens of block i, h_{i-1})
        with h_{-1} = 0.  When h_i is in hash_to_block_id and the block holds the same
        token ids, the block is shared (one more reference); otherwise a new block is
        taken and registered under h_i.  The partial last block is always new and not
        registered.  All or nothing.  Returns (row padded with -1, number of hits).
        """
        tokens = [int(t) for t in tokens]
        n_full = len(tokens) // block_size
        n_blocks = -(-len(tokens) // block_size)
        if n_blocks > width:
            raise ValueError("request longer than the table width")
        plan, h = [], 0
        for i in range(n_full):
            chunk = tokens[i * block_size:(i + 1) * block_size]
            h = block_hash(chunk, h)
            hit = self.hash_to_block.get(h)
            if hit is not None and self.block_tokens[hit] != chunk:
                hit = None                  # a hash collision: not the same tokens
            plan.append((h, chunk, hit))
        misses = sum(1 for _, _, hit in plan if hit is None) + (n_blocks - n_full)
        if misses > len(self.free):
            raise OutOfBlocks(f"need {misses} blocks, {len(self.free)} free")
        row, hits = [-1] * width, 0
        for i, (h, chunk, hit) in enumerate(plan):
            if hit is not None:
                self.incref(hit)
                row[i] = hit
                hits += 1
            else:
                b = self.alloc(1)[0]
                if h in self.hash_to_block:          # collision: the newer block takes the hash
                    self._forget(self.hash_to_block[h])
                self.hash_to_block[h] = b
                self.block_hash[b] = h
                self.block_tokens[b] = chunk
                row[i] = b
        if n_blocks > n_full:
            row[n_full] = self.alloc(1)[0]
        return row, hits

    def release_table(self, row) -> None:
        """End of a request: walk its table in reverse (题目6, step 4) and drop one
        reference per assigned entry."""
        for block in reversed([int(x) for x in row]):
            if block >= 0:
                self.decref(block)

    def share(self, row) -> list[int]:
        """A second table that points at the same blocks (§11.3 sharing): a copy of
        ``row`` with one more reference on every assigned entry."""
        out = [int(x) for x in row]
        for block in out:
            if block >= 0:
                self.incref(block)
        return out

    def prepare_write(self, row: list[int], start: int, count: int, block_size: int):
        """Make logical positions [start, start+count) writable for this table.

        Each logical block they touch must be assigned and private: an unassigned
        entry (-1) gets a new block (题目4, on-demand growth); an entry whose block is
        shared (refs > 1) gets copy-on-write (§11.3): a new block is allocated, the
        data is to be copied from the old one, and the old block loses this
        table's reference.  Returns the (src, dst) copy pairs in logical-block
        order.  All or nothing: when the free stack is too short nothing changes.
        """
        if count <= 0:
            return []
        first = start // block_size
        last = (start + count - 1) // block_size
        if last >= len(row):
            raise ValueError("positions beyond the table width")
        need = sum(1 for lb in range(first, last + 1) if row[lb] < 0 or self.refs[row[lb]] > 1)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        copies = []
        for lb in range(first, last + 1):
            old = row[lb]
            if old < 0:
                row[lb] = self.alloc(1)[0]
            elif self.refs[old] > 1:
                new = self.alloc(1)[0]
                self.decref(old)
                row[lb] = new
                copies.append((old, new))
            else:
                self._forget(old)   # a private block about to change no longer matches its hash
        return copies


# --------------------------------------------------------------------------------------
# prefix-cache hash (题目6 leaves compute_hash open; this is FNV-1a 64, chained)
# --------------------------------------------------------------------------------------

def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """FNV-1a, 64-bit: for each byte, xor it in, then multiply by the FNV prime."""
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(tokens, prefix_hash: int) -> int:
    """Hash of one full block chained on the previous block's hash: FNV-1a 64 over the
    previous hash (8 bytes, little-endian) followed by each token id (4 bytes, LE)."""
    data = int(prefix_hash).to_bytes(8, "little") + b"".join(
        int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)


# --------------------------------------------------------------------------------------
# metadata builders
# --------------------------------------------------------------------------------------

def slot_mapping(table, block_size: int, seq_idx, positions) -> list[int]:
    """Slot of each written token: table[seq][p // B] * B + p mod B ("从零开始写Qwen3（六）",
    分页自注意力的改进 address rule and the precomputed slot_mapping of 自己来实现).
    A token whose block is unassigned gets -1 (skipped by the write)."""
    out = []
    for s, p in zip(seq_idx, positions):
        phys = int(table[int(s)][int(p) // block_size])
        out.append(phys * block_size + int(p) % block_size if phys >= 0 else -1)
    return out


def cu_seqlens(lengths) -> tuple[list[int], int]:
    """Packed-batch prefix sums ("Sayfalı dikkat", Değişken uzunluklu yol): batch+1
    entries starting at 0 and ending at the total, plus the maximum length."""
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return cu, max([int(n) for n in lengths], default=0)


def request_index(cu) -> list[int]:
    """Which request every packed token belongs to (the same example's index lists)."""
    out = []
    for i in range(len(cu) - 1):
        out.extend([i] * (cu[i + 1] - cu[i]))
    return out


# --------------------------------------------------------------------------------------
# sizing ("Paged attention 与 online softmax" §11.1; "从零开始写Qwen3（六）" KVCache大小计算)
# --------------------------------------------------------------------------------------

def blocks_per_layer(tokens: int, block_size: int) -> int:
    return ceil_div(tokens, block_size)


def total_blocks(tokens: int, block_size: int, layers: int) -> int:
    return layers * blocks_per_layer(tokens, block_size)


def block_bytes(block_size: int, kv_dim: int, elem_bytes: int) -> int:
    """One block holds B tokens of K and of V: B * 2 * kvDim * element size."""
    return block_size * 2 * kv_dim * elem_bytes


def pool_bytes(num_blocks: int, block_size: int, kv_dim: int, elem_bytes: int) -> int:
    return num_blocks * block_bytes(block_size, kv_dim, elem_bytes)


def last_block_fill(tokens: int, block_size: int) -> int:
    """Slots used in the last block: T - B * (ceil(T/B) - 1)."""
    return tokens - block_size * (blocks_per_layer(tokens, block_size) - 1)


def kv_bytes_per_token(layers: int, kv_dim: int, elem_bytes: int) -> int:
    """K and V of every layer for one token: 2 * L * kvDim * element size."""
    return 2 * layers * kv_dim * elem_bytes


def contiguous_waste(used, max_len: int) -> tuple[int, int]:
    """Pre-allocating max_len tokens per request (题目4 part 1): (allocated, wasted)."""
    alloc = max_len * len(used)
    return alloc, alloc - sum(used)


def paged_waste(used, block_size: int) -> tuple[int, int]:
    """Allocating whole blocks on demand (题目4 part 2): (allocated, wasted) tokens."""
    alloc = sum(ceil_div(u, block_size) * block_size for u in used)
    return alloc, alloc - sum(used)

"""CPU oracle of the host block manager with prefix caching (test infrastructure only; see the
package docstring).

Follows the MinivLLM guide "vLLM 技术路线", Step 3 §3.2 (Block: reference count, content hash
of a full block chained with the previous block's hash, cache-miss test "not found, or the
cached block's tokens differ") and §3.3 (BlockManager: can_allocate / allocate_with_cache /
can_append / append / deallocate), and Step 4 §4.5 (prepare_prefill writes only the uncached
tokens; prepare_decode's new slot is ``block_table[-1] * block_size + last_block_num_tokens - 1``;
the 257th token of a 256-token block opens a new block).

Readings where the pages leave a step open (the same ones the C++ manager documents):

* hash of a full block: 64-bit FNV-1a over the previous block's hash (8 bytes, little endian;
  omitted for the first block) followed by the block's token ids (4 bytes each, little
  endian), masked to ``hash_bits`` bits (64 = unmasked; fewer bits only to force collisions);
* free blocks form a FIFO list, initially 0 .. num_blocks-1; allocation takes the head, a
  freed block goes to the tail; a freed block keeps its hash and tokens (still findable) until
  it is handed out again, at which point its old hash entry is dropped;
* ``allocate`` walks the prompt's blocks; a full block hits when its hash is registered and the
  registered block holds exactly these tokens; the first miss makes every later block a miss;
  a hit on a block in use adds a reference, a hit on a free block takes it off the free list
  (reference count 1, contents kept); missed full blocks get a fresh block and register their
  hash; the partial last block is never hashed or shared;
* ``can_allocate`` needs as many free blocks as the sequence has blocks (hits not counted);
* ``append`` runs after the new token was added: length % block_size == 1 takes a new block,
  == 0 hashes and registers the now-full last block;
* ``deallocate`` drops one reference per table entry, last block first; a block reaching zero
  goes to the tail of the free list.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """64-bit FNV-1a: for each byte, xor it in, then multiply by the FNV prime (mod 2^64)."""
    for b in data:
        h ^= b
        h = (h * FNV_PRIME) & MASK64
    return h


def block_hash(tokens, prefix: int, hash_bits: int = 64) -> int:
    """Hash of one full block chained with its predecessor's hash (-1 = first block)."""
    data = b""
    if prefix != -1:
        data += int(prefix).to_bytes(8, "little")
    for t in tokens:
        data += (int(t) & 0xFFFFFFFF).to_bytes(4, "little")
    h = fnv1a64(data)
    return h if hash_bits >= 64 else h & ((1 << hash_bits) - 1)


class Block:
    def __init__(self, block_id: int):
        self.block_id = block_id
        self.ref_count = 0
        self.hash = -1
        self.token_ids: List[int] = []


class Sequence:
    def __init__(self, seq_id: int, tokens):
        self.seq_id = seq_id
        self.token_ids = [int(t) for t in tokens]
        self.block_table: List[int] = []
        self.num_cached_tokens = 0


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, hash_bits: int = 64):
        self.block_size = block_size
        self.hash_bits = hash_bits
        self.blocks = [Block(i) for i in range(num_blocks)]
        self.free = deque(range(num_blocks))
        self.used = set()
        self.hash_to_block: Dict[int, int] = {}
        self.seqs: Dict[int, Sequence] = {}

    # -- helpers ---------------------------------------------------------------------------
    def _num_blocks(self, n_tokens: int) -> int:
        return -(-n_tokens // self.block_size)

    def _take(self, block_id: int) -> Block:
        """Hand out `block_id` (must be free) for new contents."""
        self.free.remove(block_id)
        blk = self.blocks[block_id]
        if blk.hash != -1 and self.hash_to_block.get(blk.hash) == block_id:
            del self.hash_to_block[blk.hash]
        blk.ref_count = 1
        blk.hash = -1
        blk.token_ids = []
        self.used.add(block_id)
        return blk

    def _register(self, blk: Block, h: int, tokens) -> None:
        blk.hash = h
        blk.token_ids = list(tokens)
        self.hash_to_block[h] = blk.block_id

    # -- the manager's operations -----------------------------------------------------------
    def can_allocate(self, n_tokens: int) -> bool:
        return len(self.free) >= self._num_blocks(n_tokens)

    def allocate(self, seq_id: int, tokens) -> int:
        """allocate_with_cache: table for a new sequence; returns its cached-token count."""
        if seq_id in self.seqs:
            raise ValueError("sequence already allocated")
        seq = Sequence(seq_id, tokens)
        if not self.can_allocate(len(seq.token_ids)):
            raise MemoryError("not enough free blocks")
        bs = self.block_size
        prefix = -1
        miss = False
        for i in range(self._num_blocks(len(seq.token_ids))):
            toks = seq.token_ids[i * bs:(i + 1) * bs]
            full = len(toks) == bs
            h = block_hash(toks, prefix, self.hash_bits) if full else -1
            bid = self.hash_to_block.get(h, -1) if full else -1
            if bid == -1 or self.blocks[bid].token_ids != toks:
                miss = True
            if miss:
                blk = self._take(self.free[0])
                if full:
                    self._register(blk, h, toks)
            else:
                seq.num_cached_tokens += bs
                blk = self.blocks[bid]
                if bid in self.used:
                    blk.ref_count += 1
                else:
                    self.free.remove(bid)
                    blk.ref_count = 1
                    self.used.add(bid)
            seq.block_table.append(blk.block_id)
            prefix = h
        self.seqs[seq_id] = seq
        return seq.num_cached_tokens

    def can_append(self, seq_id: int) -> bool:
        """Room for one more token: a new block is needed when the next token opens one."""
        seq = self.seqs[seq_id]
        need = 1 if len(seq.token_ids) % self.block_size == 0 else 0
        return len(self.free) >= need

    def append(self, seq_id: int, token: int) -> None:
        """Add one token; take a block when it opens one, hash the last block when it fills it."""
        seq = self.seqs[seq_id]
        if not self.can_append(seq_id):
            raise MemoryError("no free block")
        seq.token_ids.append(int(token))
        n = len(seq.token_ids)
        bs = self.block_size
        if (n - 1) % bs == 0:  # the new token is the first of a block
            blk = self._take(self.free[0])
            seq.block_table.append(blk.block_id)
        if n % bs == 0:  # the new token fills the last block
            last = self.blocks[seq.block_table[-1]]
            prefix = self.blocks[seq.block_table[-2]].hash if len(seq.block_table) > 1 else -1
            toks = seq.token_ids[n - bs:n]
            self._register(last, block_hash(toks, prefix, self.hash_bits), toks)

    def deallocate(self, seq_id: int) -> None:
        seq = self.seqs.pop(seq_id)
        for bid in reversed(seq.block_table):
            blk = self.blocks[bid]
            blk.ref_count -= 1
            if blk.ref_count == 0:
                self.used.discard(bid)
                self.free.append(bid)

    # -- per-step index tensors (Step 4 §4.5) ------------------------------------------------
    def block_table(self, seq_id: int) -> List[int]:
        return list(self.seqs[seq_id].block_table)

    def decode_slot(self, seq_id: int) -> int:
        """Slot of the sequence's last token: table[-1] * block_size + last_block_num_tokens - 1."""
        seq = self.seqs[seq_id]
        n = len(seq.token_ids)
        last_block_num_tokens = n - (len(seq.block_table) - 1) * self.block_size
        return seq.block_table[-1] * self.block_size + last_block_num_tokens - 1

    def prefill_slots(self, seq_id: int) -> List[int]:
        """Slots of the uncached tokens num_cached_tokens .. len-1, in order."""
        seq = self.seqs[seq_id]
        bs = self.block_size
        return [seq.block_table[p // bs] * bs + p % bs
                for p in range(seq.num_cached_tokens, len(seq.token_ids))]

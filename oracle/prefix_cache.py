"""Oracle prefix cache on top of the oracle block manager.  Plain Python.

From the pages:

* A full block is identified by a chained hash: SHA-256 over the parent
  block's hash, the block's own token ids and an extra key (say, an adapter
  id), so blocks match only when the whole prefix before them matches
  (vLLM's PagedAttention: How Memory Management Supports Large Model
  Inference, "2.4"; PagedAttention (tensortonic), "8. Reusing Work Across
  Separate Requests").  Only full blocks are cached.
* A map from hash to block serves lookups; a new request compares its prompt
  block by block and takes every matching block (count + 1) up to the first
  miss; even if the whole prompt matches, its last token is computed again
  ("2.4").
* Freed blocks go to the back of the free queue and keep their entries;
  allocation takes the front block and, if it still carries an entry, drops
  it: the queue order is the eviction order ("2.4"; "7", step 5).

Choices where the pages are silent (the library follows the same ones):

* Byte encoding of a hash input: the parent hash (32 zero bytes for the
  first block), then the block's token ids as int32 little-endian, then the
  extra key's bytes.
* A sequence returns its blocks to the free queue last block first, so its
  leading blocks (the shared prefix) are evicted last.
* When two blocks end up with the same hash (a block copied on write), the
  first one keeps the entry.
* Appends without token ids (``append``, ``append_batch``) leave the
  sequence's later blocks unhashed.
* Swapping a block out drops its entry; swapping the sequence back in enters
  its full blocks again.
"""

from __future__ import annotations

import hashlib

from .block_manager import BlockManager


def chain_hash(parent: bytes | None, tokens, extra: bytes = b"") -> bytes:
    """SHA-256(parent || int32 little-endian tokens || extra), hashlib's."""
    body = b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return hashlib.sha256((parent or bytes(32)) + body + bytes(extra)).digest()


class CachingBlockManager(BlockManager):
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self.by_hash: dict[bytes, int] = {}
        self.hash_of: dict[int, bytes] = {}  # block -> its entry in by_hash
        self.tokens: dict = {}
        self.hashes: dict = {}
        self.extra: dict = {}
        self.hash_ok: dict = {}

    # -- queries ----------------------------------------------------------------
    def num_cached_blocks(self) -> int:
        return len(self.by_hash)

    def block_hash(self, seq, j: int) -> bytes:
        return self.hashes[seq][j]

    def cached_block(self, h: bytes) -> int:
        return self.by_hash.get(h, -1)

    # -- the cache ----------------------------------------------------------------
    def _forget(self, b: int) -> None:
        h = self.hash_of.pop(b, None)
        if h is not None and self.by_hash.get(h) == b:
            del self.by_hash[h]

    def _remember(self, b: int, h: bytes) -> None:
        if h in self.by_hash or b in self.hash_of:
            return
        self.by_hash[h] = b
        self.hash_of[b] = h

    def _pop_free(self) -> int:
        b = self.free.popleft()
        self._forget(b)
        return b

    def _release_order(self, table):
        return list(reversed(table))

    def _on_swap_out(self, b: int) -> None:
        self._forget(b)

    def _on_swap_in(self, seq) -> None:
        if not self.hash_ok.get(seq):
            return
        full = self.ntok[seq] // self.block_size
        for j, h in enumerate(self.hashes[seq][:full]):
            self._remember(self.tables[seq][j], h)

    # -- operations -----------------------------------------------------------------
    def add_seq(self, seq) -> None:
        super().add_seq(seq)
        self.tokens[seq], self.hashes[seq], self.extra[seq], self.hash_ok[seq] = [], [], b"", True

    def add_seq_cached(self, seq, tokens, extra: bytes = b"") -> int:
        """Start ``seq`` from its prompt; returns the tokens already cached."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        table, hashes = [], []
        parent = None
        for j in range(len(tokens) // bs):
            h = chain_hash(parent, tokens[j * bs:(j + 1) * bs], extra)
            b = self.by_hash.get(h)
            if b is None:
                break
            if self.ref[b] == 0:
                if b in self.free:
                    self.free.remove(b)
                else:
                    self.held.remove(b)
            self.ref[b] += 1
            table.append(b)
            hashes.append(h)
            parent = h
        n = len(table) * bs
        if n == len(tokens) and n > 0:
            n -= 1  # the last token is computed even on a full hit
        self.tables[seq] = table
        self.ntok[seq] = n
        self.tokens[seq] = tokens[:n]
        self.hashes[seq] = hashes
        self.extra[seq] = bytes(extra)
        self.hash_ok[seq] = True
        return n

    def append(self, seq, n: int) -> list[int]:
        slots = super().append(seq, n)  # all or nothing: a refused append changes nothing
        if n > 0:
            self.hash_ok[seq] = False
        return slots

    def append_tokens(self, seq, tokens) -> list[int]:
        tokens = [int(t) for t in tokens]
        ok = self.hash_ok[seq]
        slots = super().append(seq, len(tokens))  # all or nothing
        if not ok:
            return slots
        toks = self.tokens[seq]
        bs = self.block_size
        for t in tokens:
            toks.append(t)
            if len(toks) % bs == 0:
                j = len(toks) // bs - 1
                if j >= len(self.hashes[seq]):
                    parent = self.hashes[seq][j - 1] if j else None
                    self.hashes[seq].append(chain_hash(parent, toks[j * bs:(j + 1) * bs], self.extra[seq]))
                self._remember(self.tables[seq][j], self.hashes[seq][j])
        return slots

    def append_batch(self, seqs) -> list[int]:
        seqs = list(seqs)
        slots = super().append_batch(seqs)
        for q in seqs:
            self.hash_ok[q] = False
        return slots

    def fork(self, parent, child) -> None:
        super().fork(parent, child)
        self.tokens[child] = list(self.tokens[parent])
        self.hashes[child] = list(self.hashes[parent])
        self.extra[child] = self.extra[parent]
        self.hash_ok[child] = self.hash_ok[parent]

    def free_seq(self, seq) -> None:
        super().free_seq(seq)
        for d in (self.tokens, self.hashes, self.extra, self.hash_ok):
            d.pop(seq, None)

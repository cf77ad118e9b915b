"""Oracle block manager: free list, reference counts, copy-on-write.  Plain Python.

Rules, each from the pages:

* The pool is a fixed set of physical blocks handed out on demand; a free
  block fits any request (PagedAttention and vLLM: Paging the KV Cache Like an
  OS, "Step 2"; Batching and PagedAttention, "How PagedAttention virtualizes
  the KV cache").  The free list is a FIFO queue seeded with a given order
  (vLLM's PagedAttention: How Memory Management Supports Large Model
  Inference, "7": a deque over the block ids).
* Logical block j holds positions 16j..16j+15; a new block is taken only when
  the last one is full (Paging the KV Cache Like an OS, "Step 3", request A).
* Each block carries a reference count; a forked sequence copies its parent's
  table and bumps the counts; when a count reaches zero the block returns to
  the pool (Paging the KV Cache Like an OS, "Step 4", beam search).
* Copy-on-write: writing into a partly filled last block whose count is above
  one allocates a fresh block, records a copy (src, dst), repoints the
  writer's table and lowers the original's count; a writer that finds the
  count at one writes in place (Paging the KV Cache Like an OS, "Step 4",
  parallel sampling).  Full blocks are never copied (PagedAttention
  (tensortonic), "7. Sharing a Prefix Without Overwriting It").
* All or nothing: an append that cannot get every block it needs changes
  nothing (Paging the KV Cache Like an OS, "Step 2", fourth difference).

* Swapping: a group of sequences (e.g. the beams of one request) is evicted
  whole; each distinct block of the group moves to a host block and back
  into a fresh device block later, blocks shared inside the group staying
  shared (PagedAttention: Virtual Memory for the KV Cache, "Scheduling and
  preemption").  A group whose blocks are shared outside it is refused.

Choices of this implementation, where the pages are silent:

* A freed sequence returns its blocks in table order to the back of the queue.
* A block named by a copy that has not been handed out yet (``take_copies``)
  is held back from the free list until that hand-out, so no block is reused
  as a copy destination (or overwritten) before its pending copy runs.
* Swap pairs are listed in order of first appearance (sequence order, then
  table order); host blocks come from their own FIFO list; a swap-out waits
  for pending copy-on-write copies to be taken.
"""

from __future__ import annotations

from collections import deque


class NoFreeBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        self.free = deque(order)
        assert sorted(self.free) == list(range(num_blocks))
        self.ref = [0] * self.num_blocks
        self.tables: dict[int, list[int]] = {}
        self.ntok: dict[int, int] = {}
        self.pending: list[tuple[int, int]] = []
        self.held: list[int] = []
        self.swapped: set = set()
        self.host_free: deque = deque()
        self.host_ref: list[int] = []

    # -- queries -------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def table(self, seq) -> list[int]:
        return list(self.tables[seq])

    def num_tokens(self, seq) -> int:
        return self.ntok[seq]

    def refcount(self, block: int) -> int:
        return self.ref[block]

    # -- operations ----------------------------------------------------------
    def add_seq(self, seq) -> None:
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.ntok[seq] = 0

    def _blocks_for(self, ntok: int) -> int:
        return -(-ntok // self.block_size)

    def append(self, seq, n: int) -> list[int]:
        """Reserve slots for n more tokens; returns their slots (block*bs+off)."""
        if seq in self.swapped:
            raise ValueError(f"sequence {seq} is swapped out")
        table = self.tables[seq]
        T = self.ntok[seq]
        bs = self.block_size
        new_blocks = self._blocks_for(T + n) - self._blocks_for(T)
        cow = n > 0 and T % bs != 0 and self.ref[table[-1]] > 1
        if len(self.free) < new_blocks + int(cow):
            raise NoFreeBlocks(f"need {new_blocks + int(cow)}, have {len(self.free)}")
        if cow:
            src = table[-1]
            dst = self._pop_free()
            self.pending.append((src, dst))
            self.ref[src] -= 1
            self.ref[dst] = 1
            table[-1] = dst
        slots = []
        for _ in range(n):
            if T % bs == 0:
                b = self._pop_free()
                self.ref[b] = 1
                table.append(b)
            slots.append(table[T // bs] * bs + T % bs)
            T += 1
        self.ntok[seq] = T
        return slots

    def append_batch(self, seqs) -> list[int]:
        """One token for each sequence, all or nothing over the batch."""
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence appears twice in the batch")
        if any(q in self.swapped for q in seqs):
            raise ValueError("a sequence of the batch is swapped out")
        need = 0
        bs = self.block_size
        ref = {}
        for s in seqs:
            T = self.ntok[s]
            if T % bs == 0:
                need += 1
                continue
            last = self.tables[s][-1]
            r = ref.get(last, self.ref[last])
            if r > 1:  # this writer copies; the next sharer sees one fewer
                need += 1
                ref[last] = r - 1
        if len(self.free) < need:
            raise NoFreeBlocks(f"need {need}, have {len(self.free)}")
        return [self.append(s, 1)[0] for s in seqs]

    def fork(self, parent, child) -> None:
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        if parent in self.swapped:
            raise ValueError(f"sequence {parent} is swapped out")
        table = self.tables[parent]
        for b in table:
            self.ref[b] += 1
        self.tables[child] = list(table)
        self.ntok[child] = self.ntok[parent]

    def _in_pending(self, b: int) -> bool:
        return any(b == s or b == d for s, d in self.pending)

    def _pop_free(self) -> int:
        return self.free.popleft()

    def _release(self, b: int) -> None:
        if self._in_pending(b):
            self.held.append(b)
        else:
            self.free.append(b)

    def _release_order(self, table):
        return table

    def free_seq(self, seq) -> None:
        table = self.tables.pop(seq)
        del self.ntok[seq]
        if seq in self.swapped:
            self.swapped.discard(seq)
            for h in table:
                self.host_ref[h] -= 1
                if self.host_ref[h] == 0:
                    self.host_free.append(h)
            return
        for b in self._release_order(table):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self._release(b)

    def take_copies(self) -> list[tuple[int, int]]:
        pairs = self.pending
        self.pending = []
        for b in self.held:
            if self.ref[b] == 0:
                self.free.append(b)
        self.held = []
        return pairs

    # -- swapping (PagedAttention: Virtual Memory for the KV Cache, "Scheduling
    # and preemption": a group is evicted whole; its blocks go to CPU memory and
    # come back later) ----------------------------------------------------------
    def set_host_blocks(self, n: int) -> None:
        assert not self.swapped
        self.host_free = deque(range(n))
        self.host_ref = [0] * n

    def _group(self, seqs, want_swapped):
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence appears twice in the group")
        uses: dict[int, int] = {}
        order: list[int] = []
        for q in seqs:
            if q not in self.tables:
                raise KeyError(q)
            if (q in self.swapped) != want_swapped:
                raise ValueError(f"sequence {q} is in the wrong place for this swap")
            for b in self.tables[q]:
                if b not in uses:
                    order.append(b)
                uses[b] = uses.get(b, 0) + 1
        return seqs, order, uses

    def swap_out(self, seqs) -> list[tuple[int, int]]:
        seqs, order, uses = self._group(seqs, False)
        if self.pending:
            raise ValueError("copy-on-write pairs pending")
        if any(self.ref[b] != uses[b] for b in order):
            raise ValueError("a block is shared outside the group")
        if len(self.host_free) < len(order):
            raise NoFreeBlocks("host pool")
        pairs, where = [], {}
        for b in order:
            h = self.host_free.popleft()
            self.host_ref[h] = self.ref[b]
            self.ref[b] = 0
            self._on_swap_out(b)
            self.free.append(b)
            where[b] = h
            pairs.append((b, h))
        for q in seqs:
            self.tables[q] = [where[b] for b in self.tables[q]]
            self.swapped.add(q)
        return pairs

    def swap_in(self, seqs) -> list[tuple[int, int]]:
        seqs, order, uses = self._group(seqs, True)
        if any(self.host_ref[h] != uses[h] for h in order):
            raise ValueError("a host block is shared outside the group")
        if len(self.free) < len(order):
            raise NoFreeBlocks("device pool")
        pairs, where = [], {}
        for h in order:
            b = self._pop_free()
            self.ref[b] = self.host_ref[h]
            self.host_ref[h] = 0
            self.host_free.append(h)
            where[h] = b
            pairs.append((h, b))
        for q in seqs:
            self.tables[q] = [where[h] for h in self.tables[q]]
            self.swapped.discard(q)
            self._on_swap_in(q)
        return pairs

    def _on_swap_out(self, b: int) -> None:
        pass

    def _on_swap_in(self, seq) -> None:
        pass

    def is_swapped(self, seq) -> bool:
        return seq in self.swapped

    # -- helpers for tests ------------------------------------------------------
    def replay(self, ops) -> None:
        for op in ops:
            if op[0] == "add":
                self.add_seq(op[1])
            elif op[0] == "append":
                self.append(op[1], op[2])
            elif op[0] == "fork":
                self.fork(op[1], op[2])
            elif op[0] == "free":
                self.free_seq(op[1])
            else:
                raise ValueError(op)

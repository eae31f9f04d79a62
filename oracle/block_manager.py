"""Host block manager of a paged KV cache (test infrastructure; see oracle/__init__).

State, as the pages define it:

* a free list of physical block ids, first-in first-out: allocation takes from
  the front, release appends to the back ([BT] §05);
* a reference count per physical block ([KVM] CoW branching; [BT] §08);
* per sequence, a block table mapping logical block j to a physical block and a
  length in tokens ([BT] §03, §06).

Operations:

* ``append``: for each new token, j = len // B and r = len % B.  When
  j == len(table) the previous block is full (r == 0): pop a free block and
  append it ([BT] §04; [KVM] paged KV allocation, the o = 0 case).  Otherwise the
  token goes into the existing block T[j]; if that block is shared
  (ref > 1) it is first replaced by a private copy: pop p_new, record the copy
  (T[j] -> p_new), drop one reference to the old block and set T[j] = p_new
  ([KVM] CoW branching; [BT] §08; [INF] §8.3.2).  The slot written is
  T[j] * B + r.  A batch of appends is all-or-nothing: if the free list runs dry
  the whole batch is undone and ``MemoryError`` is raised ([BT] §05 raises on an
  empty free list; [BT] §10 reserves a step's blocks atomically).
* ``fork``: the child gets a copy of the parent's table, every block in it
  gains a reference, and the child's length equals the parent's ([KVM] CoW
  branching, the three constant-time steps).
* ``release``: every block of the table loses a reference; blocks reaching zero
  return to the back of the free list in table order ([KVM] host-side
  reference-counted reclamation; [BT] §05).

* host tier ([KVM] asynchronous paged swap, Figure 11 and the three
  migration steps): ``attach_host`` gives the manager a pool of pinned host
  frames with its own free list; ``swap_out`` moves a sequence's blocks to host
  frames (the frames are taken, the data is copied, the table entries are
  re-tagged as host-resident with their frame index, the device blocks go back
  to the free list); ``swap_in`` takes fresh device blocks for the host entries
  and gives the frames back.  The table is the pages' extended block table:
  every entry carries its residency, ``("hbm", block)`` or ``("host", frame)``.

Readings where the pages are open: FIFO discipline (the runnable teaching code
of [BT] §05 is FIFO; [KVM] also says ring buffer or stack/FIFO); within a batch,
sequences are served in the order given and each sequence's tokens
consecutively; the copy covers the whole block (the contents beyond the
sequence's length are never read).  For the host tier: only the blocks the
sequence holds alone (reference count 1) move, in table order; a block it
shares with a fork or the prefix cache stays in HBM with the sequence's
reference, since the other holders still read it; frames come from the front
of a FIFO host free list and go back to its back; swap_in takes device blocks
from the front of the free list in table order, all or nothing, like an
append; a swapped-out sequence (one with a host entry) can be released but
not appended to, forked or read until it is swapped back in.
"""

from __future__ import annotations

import copy
from collections import deque


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.held = [0] * num_blocks  # references held outside the tables (a prefix cache)
        self.tables: dict = {}
        self.lengths: dict = {}
        self.host_free = None   # FIFO of free host frames once a host tier is attached
        self.n_frames = 0
        self.frames: dict = {}  # seq -> {logical block j: host frame} of its host-resident entries

    # -- sequences -------------------------------------------------------
    def add(self, seq) -> None:
        if seq in self.tables:
            raise ValueError(f"sequence {seq} already exists")
        self.tables[seq] = []
        self.lengths[seq] = 0

    def fork(self, parent, child) -> None:
        if parent not in self.tables:
            raise ValueError(f"unknown parent {parent}")
        if child in self.tables:
            raise ValueError(f"sequence {child} already exists")
        self._resident(parent)
        self.tables[child] = list(self.tables[parent])
        for p in self.tables[child]:
            self.ref[p] += 1
        self.lengths[child] = self.lengths[parent]

    def release(self, seq) -> list:
        """Drop the sequence; return the blocks that went back to the free list.  Frames of
        host-resident entries go back to the host free list, in table order."""
        if seq not in self.tables:
            raise ValueError(f"unknown sequence {seq}")
        freed = []
        host = self.frames.pop(seq, {})
        for j, p in enumerate(self.tables.pop(seq)):
            if j in host:
                self.host_free.append(host[j])
                continue
            self.ref[p] -= 1
            if self.ref[p] == 0:
                self.free.append(p)
                freed.append(p)
        del self.lengths[seq]
        return freed

    # -- host tier ---------------------------------------------------------
    def attach_host(self, n_frames: int, free_order=None) -> None:
        if self.host_free is not None:
            raise ValueError("a host tier is already attached")
        if n_frames <= 0:
            raise ValueError("n_frames must be positive")
        order = list(range(n_frames)) if free_order is None else [int(f) for f in free_order]
        if sorted(order) != list(range(n_frames)):
            raise ValueError("free_order must be a permutation of the frame ids")
        self.host_free = deque(order)
        self.n_frames = int(n_frames)

    def swapped(self, seq) -> bool:
        return bool(self.frames.get(seq))

    def _resident(self, seq) -> None:
        if seq not in self.tables:
            raise ValueError(f"unknown sequence {seq}")
        if self.swapped(seq):
            raise ValueError(f"sequence {seq} is swapped out")

    def swap_out(self, seq) -> list:
        """Move the blocks only ``seq`` holds to host frames.  Returns the (block, frame)
        copies in table order; the blocks go to the back of the free list.  All or
        nothing: MemoryError when the host free list is too short."""
        if self.host_free is None:
            raise ValueError("no host tier attached")
        self._resident(seq)
        table = self.tables[seq]
        moved = [j for j, p in enumerate(table) if self.ref[p] == 1]
        if len(moved) > len(self.host_free):
            raise MemoryError("no free host frame")
        pairs, host = [], {}
        for j in moved:
            p, f = table[j], self.host_free.popleft()
            pairs.append((p, f))
            host[j] = f
            self.ref[p] = 0
            self.free.append(p)
            table[j] = None
        if host:
            self.frames[seq] = host
        return pairs

    def swap_in(self, seq) -> list:
        """Give every host-resident entry of ``seq`` a fresh device block.  Returns the
        (frame, block) copies in table order; the frames go to the back of the host free
        list.  All or nothing: MemoryError when the free list is too short."""
        if seq not in self.tables:
            raise ValueError(f"unknown sequence {seq}")
        host = self.frames.get(seq, {})
        if len(host) > len(self.free):
            raise MemoryError("no free KV block")
        pairs = []
        table = self.tables[seq]
        for j in sorted(host):
            p = self._pop_free()
            table[j] = p
            pairs.append((host[j], p))
            self.host_free.append(host[j])
        self.frames.pop(seq, None)
        return pairs

    def residency(self, seq) -> list:
        """The extended block table of ``seq``: ("hbm", block) or ("host", frame) per entry."""
        host = self.frames.get(seq, {})
        return [("host", host[j]) if j in host else ("hbm", p) for j, p in enumerate(self.tables[seq])]

    def add_with_blocks(self, seq, blocks) -> None:
        """Register a sequence whose table starts with ``blocks`` (full blocks it shares):
        each gains a reference; the length is len(blocks) * B."""
        if seq in self.tables:
            raise ValueError(f"sequence {seq} already exists")
        self.tables[seq] = list(blocks)
        for p in blocks:
            self.ref[p] += 1
        self.lengths[seq] = len(blocks) * self.block_size

    def retain(self, blocks) -> None:
        """A holder outside the tables takes one reference on each block."""
        for p in blocks:
            if self.ref[p] <= 0:
                raise ValueError(f"block {p} is not allocated")
            self.ref[p] += 1
            self.held[p] += 1

    def drop(self, blocks) -> list:
        """The outside holder gives its references back; blocks reaching zero return
        to the back of the free list in the given order.  Returns those blocks."""
        freed = []
        for p in blocks:
            if self.held[p] <= 0:
                raise ValueError(f"block {p} is not held")
            self.held[p] -= 1
            self.ref[p] -= 1
            if self.ref[p] == 0:
                self.free.append(p)
                freed.append(p)
        return freed

    # -- growth ------------------------------------------------------------
    def _pop_free(self) -> int:
        if not self.free:
            raise MemoryError("no free KV block")
        p = self.free.popleft()
        self.ref[p] = 1
        return p

    def _append_one(self, seq, cow_pairs: list) -> int:
        table = self.tables[seq]
        length = self.lengths[seq]
        j, r = divmod(length, self.block_size)
        if j == len(table):
            table.append(self._pop_free())
        elif self.ref[table[j]] > 1:
            old = table[j]
            new = self._pop_free()
            self.ref[old] -= 1
            table[j] = new
            cow_pairs.append((old, new))
        self.lengths[seq] = length + 1
        return table[j] * self.block_size + r

    def append(self, seq_ids, counts=None):
        """Append tokens; return (slots, cow_pairs).  All-or-nothing."""
        seq_ids = list(seq_ids)
        counts = [1] * len(seq_ids) if counts is None else [int(c) for c in counts]
        if len(counts) != len(seq_ids):
            raise ValueError("seq_ids and counts differ in length")
        for s, c in zip(seq_ids, counts):
            self._resident(s)
            if c < 0:
                raise ValueError("negative token count")
        saved = (copy.copy(self.free), list(self.ref),
                 {s: list(t) for s, t in self.tables.items()}, dict(self.lengths))
        slots, pairs = [], []
        try:
            for s, c in zip(seq_ids, counts):
                for _ in range(c):
                    slots.append(self._append_one(s, pairs))
        except MemoryError:
            self.free, self.ref, self.tables, self.lengths = saved
            raise
        return slots, pairs

    # -- queries -------------------------------------------------------------
    def table(self, seq) -> list:
        self._resident(seq)
        return list(self.tables[seq])

    def length(self, seq) -> int:
        return self.lengths[seq]

    def n_free(self) -> int:
        return len(self.free)

    def n_allocated(self) -> int:
        return sum(1 for r in self.ref if r > 0)

    def n_shared(self) -> int:
        return sum(1 for r in self.ref if r > 1)

    def check(self) -> None:
        """Conservation: N_free + N_allocated = N_total and {ref > 0} = allocated ([BT] §13).

        Also: every reference count equals the number of table entries naming
        the block, no block is both free and referenced, and every table has
        exactly ceil(len / B) entries.
        """
        counted = [0] * self.num_blocks
        used_frames = []
        for seq, t in self.tables.items():
            if len(t) != -(-self.lengths[seq] // self.block_size):
                raise AssertionError(f"table of {seq} has {len(t)} entries for length {self.lengths[seq]}")
            host = self.frames.get(seq, {})
            for j, p in enumerate(t):
                if j in host:
                    if p is not None:
                        raise AssertionError(f"entry {j} of {seq} is in both tiers")
                    used_frames.append(host[j])
                else:
                    counted[p] += 1
        if self.host_free is not None:
            frames = list(self.host_free) + used_frames
            if sorted(frames) != list(range(self.n_frames)):
                raise AssertionError("host frames: free + used != all frames, or a frame is used twice")
        elif used_frames:
            raise AssertionError("host entries without a host tier")
        counted = [c + h for c, h in zip(counted, self.held)]
        if counted != self.ref:
            raise AssertionError("reference counts disagree with the tables and outside holders")
        free = set(self.free)
        if len(free) != len(self.free):
            raise AssertionError("duplicate block in the free list")
        allocated = {p for p in range(self.num_blocks) if self.ref[p] > 0}
        if free & allocated:
            raise AssertionError("a referenced block is on the free list")
        if len(self.free) + len(allocated) != self.num_blocks:
            raise AssertionError("N_free + N_allocated != N_total")

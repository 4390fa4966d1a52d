"""Reference block pool for the paged KV cache -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's CPU baseline use this
module; the library never does.  It is the plain host-side bookkeeping the
pages describe, written out in Python so that the native pool of the library
can be checked against it operation by operation.

Sources (cited by page title and section):
- "vLLM 核心工程深度剖析" (ybb.press), section 2.2, the block allocator:
  a free list of physical block numbers taken from and returned to its end,
  a reference count per block, one block table per request; `allocate`
  takes ceil(n / B) blocks, `append_slot` takes a new block only when the
  last one is full, `free` drops one reference per block and returns blocks
  whose count reaches zero to the free list.  Running out of blocks is an
  error.
- the same page, section 4.1 (beam search): `fork` gives the child a copy of
  the parent's table and one more reference on every block.
- "PagedAttention 笔记" (imreese.github.io), section on copy-on-write: a
  block referenced by more than one sequence is read-only; a sequence that
  must write into such a block takes a new block, copies the shared block
  into it, points its table entry at the new block and drops one reference
  on the old one, then writes there.

Position L of a sequence lives in block table[L // B] at offset L % B, and
its slot number is table[L // B] * B + L % B (the cache-structure page's
"writing new K/V" section).

Parity pinned: the two worked examples of the reading-notes page (shared
prompt P8 -> P2 -> P15 with branches continuing in P4 and P9; copy-on-write
of P8 into P11), stored in tests/golden/block_pool_examples.json.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(RuntimeError):
    """No free block left (the allocator's out-of-memory error)."""


class ReferencePool:
    def __init__(self, num_blocks: int, block_size: int, free_list: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # a stack: the last entry is handed out first
        self.free_list: List[int] = list(range(num_blocks)) if free_list is None else list(free_list)
        self.ref_count = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    # -- allocation ---------------------------------------------------------
    def _take(self) -> int:
        if not self.free_list:
            raise OutOfBlocks("no free block")
        b = self.free_list.pop()
        self.ref_count[b] += 1
        return b

    def add_sequence(self, seq: int, num_tokens: int) -> List[int]:
        """Blocks for a new sequence of num_tokens tokens: ceil(n / B) of them."""
        if seq in self.tables or num_tokens < 0:
            raise ValueError("sequence exists or negative length")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free_list):
            raise OutOfBlocks("not enough free blocks")
        self.tables[seq] = [self._take() for _ in range(need)]
        self.lens[seq] = num_tokens
        return list(self.tables[seq])

    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve position L = len(seq) for the next token (the length
        becomes L + 1).  Returns the token's slot and the (src, dst) block copy
        that must be done first, or None.  On OutOfBlocks nothing changes."""
        table = self.tables[seq]
        L = self.lens[seq]
        B = self.block_size
        copy = None
        if L % B == 0:
            # the last block is full (or there is none): a new block
            table.append(self._take())
        else:
            last = table[L // B]
            if self.ref_count[last] > 1:
                # shared: copy-on-write into a block of its own
                new = self._take()
                copy = (last, new)
                table[L // B] = new
                self.ref_count[last] -= 1
        self.lens[seq] = L + 1
        return table[L // B] * B + L % B, copy

    def fork(self, parent: int, child: int) -> None:
        """The child shares every block of the parent."""
        if child in self.tables:
            raise ValueError("child exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref_count[b] += 1

    def free(self, seq: int) -> None:
        for b in self.tables[seq]:
            self.ref_count[b] -= 1
            if self.ref_count[b] == 0:
                self.free_list.append(b)
        del self.tables[seq]
        del self.lens[seq]

    # -- views --------------------------------------------------------------
    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])


def copy_blocks(k_pool, v_pool, pairs) -> None:
    """Block copy: every element of block src (all KV heads) is copied to
    block dst, in both pools, for each (src, dst) pair in order (numpy
    arrays with the block index first)."""
    for src, dst in pairs:
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]

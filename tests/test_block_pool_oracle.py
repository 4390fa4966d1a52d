"""The reference block pool (oracle/block_pool.py) against the pages' worked
examples (tests/golden/block_pool_examples.json) and the invariants of the
allocator they describe."""
import numpy as np
import pytest

from oracle.block_pool import OutOfBlocks, ReferencePool, copy_blocks
from tests.conftest import golden


def stack_with_top(num_blocks, top_first):
    """A free list (stack) whose next pops are top_first[0], top_first[1], ..."""
    rest = [b for b in range(num_blocks) if b not in top_first]
    return rest + list(reversed(top_first))


def test_shared_prompt_example():
    g = golden("block_pool_examples.json")["share"]
    B = g["block_size"]
    p = ReferencePool(16, B, stack_with_top(16, g["prompt_blocks"] + [4, 9]))
    a = p.add_sequence("A", 3 * B)            # the prompt fills three blocks
    assert a == g["prompt_blocks"]
    p.fork("A", "B")
    for b in g["prompt_blocks"]:
        assert p.ref_count[b] == g["shared_ref_count"]
    slot_a, copy_a = p.append_slot("A")
    slot_b, copy_b = p.append_slot("B")
    assert p.table("A") == g["branch_a"] and p.table("B") == g["branch_b"]
    assert copy_a is None and copy_b is None   # a full block is never copied
    assert slot_a == 4 * B and slot_b == 9 * B  # position 3B, offset 0 of the new blocks
    assert p.ref_count[4] == 1 and p.ref_count[9] == 1


def test_copy_on_write_example():
    g = golden("block_pool_examples.json")["cow"]
    B = g["block_size"]
    p = ReferencePool(16, B, stack_with_top(16, [g["shared_block"], g["new_block"]]))
    p.add_sequence("B", 10)                   # a partly filled block P8
    p.fork("B", "A")
    assert p.ref_count[8] == g["ref_count_before"]
    slot, copy = p.append_slot("A")           # A appends into the shared P8
    assert copy == tuple(g["copy"])
    assert p.table("A") == [g["new_block"]]
    assert p.ref_count[8] == g["ref_count_after"] and p.ref_count[11] == 1
    assert slot == 11 * B + 10                # the new token goes to P11
    slot_b, copy_b = p.append_slot("B")       # P8 is B's alone now: written in place
    assert copy_b is None and slot_b == 8 * B + 10


def test_free_returns_blocks_only_at_zero_references():
    p = ReferencePool(8, 4)
    p.add_sequence(1, 9)                       # 3 blocks
    p.fork(1, 2)
    p.append_slot(2)                           # position 9 in a partly filled, shared block: copied
    shared = p.table(1)
    free_before = len(p.free_list)
    p.free(1)
    # the first two blocks are still referenced by sequence 2; the third was copied for 2
    assert len(p.free_list) == free_before + 1 and p.free_list[-1] == shared[2]
    p.free(2)
    assert sorted(p.free_list) == list(range(8)) and all(r == 0 for r in p.ref_count)


def test_out_of_blocks_changes_nothing():
    p = ReferencePool(2, 4)
    p.add_sequence(1, 8)
    with pytest.raises(OutOfBlocks):
        p.append_slot(1)
    assert p.lens[1] == 8 and p.table(1) == [1, 0]
    with pytest.raises(OutOfBlocks):
        p.add_sequence(2, 1)
    assert 2 not in p.tables


def test_random_operations_keep_the_invariants():
    rng = np.random.default_rng(7)
    p = ReferencePool(64, 8)
    live = []
    for step in range(3000):
        op = rng.integers(4)
        try:
            if op == 0 or not live:
                s = step
                p.add_sequence(s, int(rng.integers(0, 40)))
                live.append(s)
            elif op == 1:
                p.append_slot(live[rng.integers(len(live))])
            elif op == 2:
                p.fork(live[rng.integers(len(live))], step)
                live.append(step)
            else:
                s = live.pop(rng.integers(len(live)))
                p.free(s)
        except OutOfBlocks:
            pass
        # every block is either free or referenced, never both; counts match the tables
        refs = np.zeros(64, int)
        for t in p.tables.values():
            for b in t:
                refs[b] += 1
        assert list(refs) == p.ref_count
        assert sorted(set(p.free_list)) == sorted(p.free_list)
        assert all(p.ref_count[b] == 0 for b in p.free_list)
        assert len(p.free_list) + int(np.count_nonzero(refs)) == 64
        for s, t in p.tables.items():
            assert len(t) == -(-p.lens[s] // 8)


def test_copy_blocks_copies_whole_blocks():
    k = np.arange(5 * 2 * 3, dtype=np.float32).reshape(5, 2, 3)
    v = -k
    k0, v0 = k.copy(), v.copy()
    copy_blocks(k, v, [(1, 4), (3, 0)])
    assert np.array_equal(k[4], k0[1]) and np.array_equal(v[0], v0[3])
    assert np.array_equal(k[[1, 2, 3]], k0[[1, 2, 3]]) and np.array_equal(v[[1, 2, 3]], v0[[1, 2, 3]])

"""pkv_validate on the GPU: each contract violation planted in the tables,
lengths, slots or reference counts is reported with the count and first
offender that a host-side count of the same arrays gives; clean inputs
report nothing.  The rules: used table entries inside the pool and lengths
within the table (the cache-structure page's table walk), distinct in-pool
slots in one append ("写入新 K/V"), and no slot in a block with more than one
reference ("写时复制是正确性的边界", reading-notes page)."""
import numpy as np
import pytest

import pkv_inputs as pi

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_35_amd as pkv

    pkv.library()
    torch.cuda.set_device(0)


def pkv():
    import paged_kv_cache_35_amd as m

    return m


def cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def decode_slots(bt, sl, B):
    M = bt.shape[1]
    out = np.full(len(sl), -1, np.int64)
    for s, L in enumerate(sl):
        if L <= 0 or (L - 1) // B >= M:
            continue
        idx = (L - 1) // B
        bid = int(bt[s, idx])
        out[s] = -1 if bid < 0 else bid * B + (L - 1) % B
    return out


def host_report(bt, sl, B, nb, slots=None, ref=None):
    """The report written out on the host, one rule at a time."""
    S, M = bt.shape
    cap = M * B
    bad_len = [s for s in range(S) if sl[s] < 0 or sl[s] > cap]
    bad_id = []
    for s in range(S):
        Lc = min(max(int(sl[s]), 0), cap)
        for i in range(-(-Lc // B)):
            if not 0 <= bt[s, i] < nb:
                bad_id.append(s * M + i)
    if slots is None:
        slots = decode_slots(bt, sl, B)
    bad_slot = [t for t, x in enumerate(slots) if x >= 0 and x // B >= nb]
    seen, dup = set(), []
    for t, x in enumerate(slots):
        if x >= 0:
            if int(x) in seen:
                dup.append(t)
            seen.add(int(x))
    shared = [] if ref is None else [t for t, x in enumerate(slots) if 0 <= x and x // B < nb and ref[x // B] > 1]
    lists = (bad_len, bad_id, bad_slot, dup, shared)
    vals = [len(l) for l in lists] + [min(l) if l else -1 for l in lists]
    return dict(zip(pkv().VALIDATE_FIELDS, vals))


def run(w, bt, sl, slots=None, ref=None):
    got = pkv().validate(cuda(bt), cuda(sl), w.num_blocks, w.B, slot_mapping=None if slots is None else cuda(slots),
                         ref_counts=None if ref is None else cuda(ref))
    want = host_report(bt, sl, w.B, w.num_blocks, slots, ref)
    print(f"  report {got}", flush=True)
    assert got == want
    return got


def workload():
    return pi.make_workload(2, S=40, len_lo=1, len_hi=300)


def test_clean_inputs_report_nothing():
    w = workload()
    print("clean decode batch", flush=True)
    got = run(w, w.block_tables.copy(), w.seq_lens.copy(), ref=np.ones(w.num_blocks, np.int32))
    assert all(v == 0 for k, v in got.items() if not k.startswith("first")), got
    assert all(v == -1 for k, v in got.items() if k.startswith("first")), got


def test_planted_table_and_length_violations():
    w = workload()
    bt, sl = w.block_tables.copy(), w.seq_lens.copy()
    B, M, nb = w.B, w.M, w.num_blocks
    used = -(-sl.astype(np.int64) // B)
    bt[3, 0] = -3                           # used entry below the pool
    bt[5, used[5] - 1] = nb                 # the last used entry, one past the pool
    bt[7, 0] = nb + 100
    s_unused = int(np.argmin(used))         # an entry no length reaches: not reported
    bt[s_unused, M - 1] = -99
    sl[11] = -2                             # negative length
    sl[13] = M * B + 5                      # past the table: every entry of the row is used
    bt[13, M - 1] = nb + 1
    print(f"planted tables: M={M} nb={nb}", flush=True)
    got = run(w, bt, sl)
    assert got["bad_block_ids"] >= 4 and got["bad_seq_lens"] == 2


def test_planted_slot_violations():
    w = workload()
    g = np.random.default_rng(7)
    B, nb = w.B, w.num_blocks
    T = 600
    slots = g.choice(nb * B, size=T, replace=False).astype(np.int64)
    slots[100] = slots[20]                  # a slot three times
    slots[101] = slots[20]
    slots[300] = slots[299]
    slots[50] = nb * B + 7                  # past the pool
    slots[60] = -1                          # a skip, not an error
    ref = np.ones(nb, np.int32)
    ref[slots[400] // B] = 2                # blocks that two sequences reference
    ref[slots[10] // B] = 3
    print("planted slots", flush=True)
    got = run(w, w.block_tables, w.seq_lens, slots=slots, ref=ref)
    assert got["duplicate_slots"] == 3 and got["first_duplicate_slot"] == 100
    assert got["bad_slots"] == 1 and got["first_bad_slot"] == 50
    assert got["shared_block_writes"] >= 2


def test_forked_sequences_without_copy_on_write():
    # two sequences with the same table row and length (a fork whose last
    # block was not copied before the append): the decode step's slots
    # repeat, and both write a block that two sequences reference
    w = workload()
    bt, sl = w.block_tables.copy(), w.seq_lens.copy()
    bt[9] = bt[4]
    sl[9] = sl[4]
    ref = np.ones(w.num_blocks, np.int32)
    used = -(-int(sl[4]) // w.B)
    ref[bt[4, :used]] = 2
    print("fork without copy-on-write", flush=True)
    got = run(w, bt, sl, ref=ref)
    assert got["duplicate_slots"] == 1 and got["first_duplicate_slot"] == 9
    assert got["shared_block_writes"] == 2 and got["first_shared_block_write"] == 4


def test_many_slots_across_work_groups():
    # 5000 slots (20 work-groups of the pairwise check), repeats far apart
    w = workload()
    g = np.random.default_rng(11)
    T = 5000
    slots = g.choice(w.num_blocks * w.B, size=T, replace=False).astype(np.int64)
    for a, b in ((3, 4999), (256, 257), (1000, 4000), (1000, 4500), (255, 256)):
        slots[b] = slots[a]
    slots[g.choice(T, size=40, replace=False)] = -1
    print("5000 slots", flush=True)
    run(w, w.block_tables, w.seq_lens, slots=slots)

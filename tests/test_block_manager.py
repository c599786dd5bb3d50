"""Block manager: the reference model against a contiguous history, and the
library's native manager against the reference (host only, no device)."""

import random
import threading

import numpy as np
import pytest

import paged_kv_cache_56_amd as pkv
from oracle.block_manager import ReferenceBlockManager, PoolExhausted

BS = 16


def _random_ops(seed, n_ops=400, num_blocks=48):
    """A seeded stream of (op, args): add, fork, append batches, free."""
    rng = random.Random(seed)
    live, next_id, ops = [], 0, []
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.12 or not live:
            ops.append(("add", next_id)); live.append(next_id); next_id += 1
        elif r < 0.25:
            p = rng.choice(live)
            ops.append(("fork", p, next_id)); live.append(next_id); next_id += 1
        elif r < 0.33 and len(live) > 1:
            s = rng.choice(live); live.remove(s); ops.append(("free", s))
        else:
            k = rng.randint(1, min(4, len(live)))
            ops.append(("append", rng.sample(live, k)))
    return ops


def _run_reference(ops, num_blocks, order):
    """Runs ops on the reference, with a simulated cache: every appended token
    gets a unique value written to its slot (after the CoW copies run)."""
    ref = ReferenceBlockManager(num_blocks, BS, order)
    cache = np.full(num_blocks * BS, -1, dtype=np.int64)
    history = {}                          # the contiguous model: seq -> tokens
    trace, value = [], 0
    for op in ops:
        if op[0] == "add":
            ref.add_sequence(op[1]); history[op[1]] = []
        elif op[0] == "fork":
            ref.fork(op[1], op[2]); history[op[2]] = list(history[op[1]])
        elif op[0] == "free":
            ref.free_sequence(op[1]); del history[op[1]]
        else:
            try:
                slots, copies = ref.append_slots(op[1])
            except PoolExhausted:
                trace.append(("full",)); continue
            for s, d in copies:
                cache[d * BS:(d + 1) * BS] = cache[s * BS:(s + 1) * BS]
            for seq, slot in zip(op[1], slots):
                cache[slot] = value; history[seq].append(value); value += 1
            trace.append((tuple(slots), tuple(copies)))
    return ref, cache, history, trace


@pytest.mark.parametrize("seed", range(6))
def test_reference_never_corrupts_a_sequence(seed):
    """Read through its table, every live sequence holds exactly its own
    history (shared prefix + its own appends), whatever the others did."""
    order = list(range(48)); random.Random(seed).shuffle(order)
    ref, cache, history, _ = _run_reference(_random_ops(seed), 48, order)
    for seq, toks in history.items():
        t = ref.tables[seq]
        got = [int(cache[t[p // BS] * BS + p % BS]) for p in range(len(toks))]
        assert got == toks
    # bookkeeping invariants: references match the tables, the pool is the rest
    counts = np.zeros(48, int)
    for t in ref.tables.values():
        for b in t:
            counts[b] += 1
    assert list(counts) == ref.ref
    assert sorted(ref.free + [b for b in range(48) if counts[b]]) == list(range(48))


def test_reference_cow_only_for_shared_partial_blocks():
    ref = ReferenceBlockManager(8, BS)
    ref.add_sequence(0)
    for _ in range(20):
        ref.append_slots([0])
    ref.fork(0, 1)
    assert ref.ref[:2] == [2, 2]
    slots, copies = ref.append_slots([1])       # partial shared block -> copy
    assert copies == [(1, 2)] and slots == [2 * BS + 4]
    slots, copies = ref.append_slots([0])       # the parent's block is private again
    assert copies == [] and slots == [1 * BS + 4]
    assert ref.ref[:3] == [2, 1, 1]
    for _ in range(11):
        ref.append_slots([0])
    slots, copies = ref.append_slots([0])       # block full: a fresh block, no copy
    assert copies == [] and slots == [3 * BS]


@pytest.mark.parametrize("seed", range(6))
def test_native_manager_matches_reference(seed):
    order = list(range(48)); random.Random(seed).shuffle(order)
    ops = _random_ops(seed)
    ref, _, _, trace = _run_reference(ops, 48, order)
    bm = pkv.BlockManager(48, free_order=order)
    k = 0
    for op in ops:
        if op[0] == "add":
            bm.add_sequence(op[1])
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        elif op[0] == "free":
            bm.free_sequence(op[1])
        else:
            try:
                slots, copies = bm.append_slots(op[1])
                got = (tuple(slots), tuple(copies))
            except pkv.PagedKVError as e:
                assert e.status == -6
                got = ("full",)
            assert got == trace[k]
            k += 1
    assert bm.num_free() == ref.num_free()
    assert [bm.refcount(b) for b in range(48)] == ref.ref
    live = sorted(ref.tables)
    tables, lens = bm.block_tables(live, 48)
    for i, s in enumerate(live):
        assert list(tables[i, : len(ref.tables[s])]) == ref.tables[s]
        assert int(lens[i]) == ref.lens[s]
        assert (tables[i, len(ref.tables[s]):] == -1).all()


def test_native_manager_errors():
    with pytest.raises(ValueError):
        pkv.BlockManager(4, free_order=[0, 0, 1, 2])
    bm = pkv.BlockManager(2)
    bm.add_sequence(7)
    with pytest.raises(pkv.PagedKVError) as e:
        bm.add_sequence(7)
    assert e.value.status == -7
    with pytest.raises(pkv.PagedKVError):
        bm.fork(99, 1)
    with pytest.raises(pkv.PagedKVError):
        bm.append_slots([7, 7])
    bm.add_sequence(8)
    bm.add_sequence(9)
    bm.append_slots([7, 8])
    with pytest.raises(pkv.PagedKVError) as e:          # pool empty: nothing changes
        bm.append_slots([9])
    assert e.value.status == -6 and bm.num_free() == 0
    tables, lens = bm.block_tables([9], 4)
    assert int(lens[0]) == 0 and (tables == -1).all()
    bm.free_sequence(7)
    assert bm.num_free() == 1
    bm.append_slots([9])


def test_native_manager_is_thread_safe():
    """Many threads fork and free children of one parent at once; at the end
    every reference is back where it started."""
    bm = pkv.BlockManager(64)
    bm.add_sequence(0)
    for _ in range(40):
        bm.append_slots([0])
    before = [bm.refcount(b) for b in range(64)]

    def worker(base):
        for i in range(200):
            c = base * 1000 + i
            bm.fork(0, c)
            bm.free_sequence(c)

    th = [threading.Thread(target=worker, args=(k + 1,)) for k in range(8)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert [bm.refcount(b) for b in range(64)] == before
    assert bm.num_free() == 64 - 3


MANAGER_MUTANTS = {
    "copy_not_recorded": ("copies.append((t[-1], b))", "pass"),
    "old_block_keeps_reference": ("                self.ref[t[-1]] -= 1\n", "                pass\n"),
    "no_copy_on_write": ("elif self.ref[t[-1]] > 1:", "elif False:"),
    "fork_without_reference": ("            self.ref[b] += 1\n", "            pass\n"),
}


@pytest.mark.parametrize("name", sorted(MANAGER_MUTANTS))
def test_planted_manager_mistake_is_caught(name, monkeypatch):
    import inspect
    import types
    import oracle.block_manager as bmmod
    src = inspect.getsource(bmmod)
    old, new = MANAGER_MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("mutant_" + name)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    monkeypatch.setitem(globals(), "ReferenceBlockManager", mod.ReferenceBlockManager)
    monkeypatch.setitem(globals(), "PoolExhausted", mod.PoolExhausted)
    caught = False
    for seed in range(6):
        try:
            test_reference_never_corrupts_a_sequence(seed)
        except (AssertionError, IndexError, ValueError):
            caught = True
            break
    assert caught, name

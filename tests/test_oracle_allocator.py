"""Pins of the oracle's block manager and pool mirror (CPU only)."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import workloads
from oracle.allocator import (AllocatorStateError, BlockAllocator, OutOfBlocks, block_hash,
                              fnv1a64, run_ops)
from oracle.expected import pool_after, stored_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_block_table_walkthrough():
    g = _golden("block_table_example.json")
    a = BlockAllocator(g["num_blocks"], g["block_size"], g["free_order"])
    cached, slots = a.allocate(0, list(range(g["prompt_len"])))
    assert cached == 0
    assert a.block_table(0) == g["table_after_prompt"]
    assert slots == g["prompt_slots"]
    got = [a.append_slot(0, 100 + i) for i in range(len(g["decode_slots"]))]
    assert got == g["decode_slots"]
    assert a.block_table(0) == g["table_after_decode"]
    assert a.take_copies() == []


def test_copy_on_write_walkthrough():
    g = _golden("cow_example.json")
    a = BlockAllocator(g["num_blocks"], g["block_size"], g["free_order"])
    a.allocate("A1", list(range(g["prompt_len"])))
    a.fork("A1", "A2")
    assert {str(b): a.ref[b] for b in a.block_table("A1")} == g["refs_after_fork"]
    for who, key in (("A1", "a1_append"), ("A2", "a2_append")):
        slot = a.append_slot(who, 0)
        assert slot == g[key]["slot"]
        assert [list(p) for p in a.take_copies()] == g[key]["copies"]
        assert a.block_table(who) == g[key]["table"]
    refs = {str(b): a.ref[b] for b in set(a.block_table("A1")) | set(a.block_table("A2"))}
    assert refs == g["refs_after"]


def test_fnv1a_published_vectors():
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_prefix_sharing_rules():
    B = 4
    a = BlockAllocator(64, B)
    base = list(range(100, 114))  # 3 full blocks + 2 tokens
    c0, s0 = a.allocate(0, base)
    assert c0 == 0
    # same first 3 full blocks -> exactly those are shared, partial block is not
    c1, s1 = a.allocate(1, base)
    t0, t1 = a.block_table(0), a.block_table(1)
    assert c1 == 12 and t0[:3] == t1[:3] and t0[3] != t1[3]
    assert [a.ref[b] for b in t0[:3]] == [2, 2, 2]
    # one token changed in block 1 breaks sharing from block 1 on, even where block 2 matches
    other = list(base); other[5] = 999
    c2, _ = a.allocate(2, other)
    t2 = a.block_table(2)
    assert c2 == 4 and t2[0] == t0[0] and len(set(t2[1:]) & set(t0)) == 0
    # freeing every holder drops the entries: a new request shares nothing
    for s in (0, 1, 2):
        a.free_seq(s)
    assert a.num_free == 64 and not a.block_of_hash
    c3, _ = a.allocate(3, base)
    assert c3 == 0
    # hashes chain on the previous block: same block content after a different prefix differs
    assert block_hash(block_hash(0, [1, 2, 3, 4]), [5, 6, 7, 8]) != block_hash(0, [5, 6, 7, 8])


def test_out_of_blocks_leaves_state_unchanged():
    a = BlockAllocator(5, 4, [4, 3, 2, 1, 0])
    a.allocate(0, list(range(8)))           # 2 blocks
    a.fork(0, 1)
    a.allocate(2, list(range(50, 61)))      # 3 blocks, pool now empty
    snap = (list(a.free), list(a.ref), {k: list(v) for k, v in a.tables.items()}, dict(a.lens))
    with pytest.raises(OutOfBlocks):
        a.allocate(3, [7])
    with pytest.raises(OutOfBlocks):
        a.append_slot(0, 1)                 # needs a new block
    with pytest.raises(OutOfBlocks):
        a.extend(2, [1, 2])                 # crosses into a new block
    assert (list(a.free), list(a.ref), {k: list(v) for k, v in a.tables.items()}, dict(a.lens)) == snap
    assert a.extend(2, [9]) == [a.block_table(2)[2] * 4 + 3]  # fits in the last block
    with pytest.raises(AllocatorStateError):
        a.fork(0, 1)
    with pytest.raises(AllocatorStateError):
        a.append_slot(42)


def _check_invariants(a: BlockAllocator):
    holders = np.zeros(a.N, dtype=np.int64)
    for seq, table in a.tables.items():
        assert len(table) == -(-a.lens[seq] // a.B)
        for b in table:
            holders[b] += 1
    assert list(holders) == a.ref
    free = list(a.free)
    assert len(free) == len(set(free))
    live = {b for t in a.tables.values() for b in t}
    assert not (live & set(free))
    assert live | set(free) == set(range(a.N))
    for b, h in a.hash_of_block.items():
        assert a.block_of_hash[h] == b and a.ref[b] > 0


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 2**31 - 1), B=st.sampled_from([1, 2, 4, 16]),
       nops=st.integers(1, 80))
def test_random_fork_prune_append_invariants(seed, B, nops):
    """Reference counts equal the number of tables holding a block; free list and
    live blocks partition the pool; after everything is freed the pool is whole."""
    rng = np.random.default_rng(seed)
    a = BlockAllocator(48, B, rng.permutation(48))
    live, nxt = [], 0
    for _ in range(nops):
        r = rng.random()
        try:
            if r < 0.25 or not live:
                n = int(rng.integers(0, 3 * B + 2))
                toks = [int(x) for x in rng.integers(0, 3, size=n)]  # small vocab: prefix hits happen
                a.allocate(nxt, toks); live.append(nxt); nxt += 1
            elif r < 0.45:
                p = live[int(rng.integers(len(live)))]
                a.fork(p, nxt); live.append(nxt); nxt += 1
            elif r < 0.8:
                s = live[int(rng.integers(len(live)))]
                a.append_slot(s, int(rng.integers(0, 3)))
            elif r < 0.9:
                s = live[int(rng.integers(len(live)))]
                a.extend(s, [int(x) for x in rng.integers(0, 3, size=int(rng.integers(1, 2 * B + 1)))])
            else:
                s = live.pop(int(rng.integers(len(live))))
                a.free_seq(s)
        except OutOfBlocks:
            pass
        _check_invariants(a)
        for src, dst in a.take_copies():
            assert src != dst
    for s in live:
        a.free_seq(s)
    assert a.num_free == a.N and sum(a.ref) == 0


def test_cow_saving_three_samples():
    """Three samples on a block-aligned prompt hold the prompt blocks once
    (count 3): 2/3 of the prompt's logical blocks need no physical block."""
    a = BlockAllocator(64, 4)
    a.allocate(0, list(range(12)))
    a.fork(0, 1); a.fork(0, 2)
    assert [a.ref[b] for b in a.block_table(0)] == [3, 3, 3]
    for s in (0, 1, 2):
        a.append_slot(s, s)
    assert a.take_copies() == []            # aligned prompt: nothing to copy
    logical = sum(len(a.block_table(s)) for s in range(3))
    physical = len({b for s in range(3) for b in a.block_table(s)})
    assert (logical, physical) == (12, 6)


@pytest.mark.parametrize("name", workloads.config_names())
def test_reassembled_pool_matches_logical_kv(name):
    """Run each small workload's op script through the reference allocator, write
    the pool mirror by the slot rule, read every sequence back through its block
    table: the result equals the generator's logical K/V exactly (for an FP8
    pool, the codes of those rows)."""
    wl = workloads.make(name, "small")
    mirror, alloc, events = pool_after(wl)
    for s in wl.decode_seqs:
        k, v = mirror.gather(alloc.block_table(s), alloc.seq_len(s))
        assert alloc.seq_len(s) == len(wl.hist[s])
        want_k, want_v = stored_rows(wl, wl.rows_k[wl.hist[s]], wl.rows_v[wl.hist[s]])
        assert np.array_equal(k, want_k)
        assert np.array_equal(v, want_v)
    _check_invariants(alloc)


def test_workload_structure():
    """Sharing and copies happen where the workloads say they do."""
    wl = workloads.make("cow", "small")
    _, alloc, events = pool_after(wl)
    assert not any(e[0] == "copy" for e in events)  # aligned prompts
    wl = workloads.make("cow504", "small")
    _, alloc, events = pool_after(wl)
    copies = [p for e in events if e[0] == "copy" for p in e[1]]
    assert len(copies) == 2 * wl.meta["groups"]    # two of three samples copy
    wl = workloads.make("prefix", "small")
    _, alloc, events = pool_after(wl)
    first = alloc.block_table(wl.decode_seqs[0])[:wl.meta["prefix_tokens"] // 16]
    for s in wl.decode_seqs:
        assert alloc.block_table(s)[:len(first)] == first
    assert all(alloc.ref[b] == len(wl.decode_seqs) for b in first)
    wl = workloads.make("beam", "small")
    _, alloc, events = pool_after(wl)
    assert any(e[0] == "copy" for e in events)


def test_generator_is_deterministic():
    for name in workloads.config_names():
        a, b = workloads.make(name, "small"), workloads.make(name, "small")
        assert np.array_equal(a.rows_k, b.rows_k) and np.array_equal(a.q, b.q)
        assert np.array_equal(a.free_order, b.free_order)
        assert len(a.ops) == len(b.ops)

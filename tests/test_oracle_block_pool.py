"""Pins for the oracle's block pool and step-input builder (CPU only).

Checked against outputs the pages print (tests/golden/), a closed form for the
number of blocks a growing sequence holds, hand-worked slot numbers, and
brute-force invariants over random operation sequences.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle.block_pool import BlockPool, PoolError, prepare_step
import oracle
from oracle import kv_bytes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pages_free_list():
    """The free list of the pages' paged_kv.py run: the generator's second draw."""
    rng = np.random.default_rng(7)
    lengths = rng.integers(50, 600, size=40)
    return lengths, rng.permutation(64)


def test_printed_block_tables_and_refcounts():
    g = json.load(open(os.path.join(GOLDEN, "paged_kv_block_tables.json")))
    _, order = _pages_free_list()
    pool = BlockPool(64, 16, free_order=order)
    a = pool.allocate(40)
    assert a == g["request_a_table"]
    b = a[:2]
    pool.share(b)
    b = b + pool.allocate(20)
    assert b == g["request_b_table"]
    shared = {str(k): v for k, v in pool.refs.items() if v > 1}
    assert shared == g["shared_ref_counts"]
    assert pool.num_free() == 64 - 5


def test_printed_waste_figures():
    g = json.load(open(os.path.join(GOLDEN, "paged_kv_block_tables.json")))
    lengths, _ = _pages_free_list()
    per_token = kv_bytes(32, 8, 128, 1, 2)
    assert per_token // 1024 == g["per_token_kib"]
    pool = BlockPool(0, 16)
    used = int(lengths.sum())
    naive = 2048 * len(lengths)
    paged = sum(pool.blocks_for(int(n)) * 16 for n in lengths)
    assert round(naive * per_token / 2**30, 2) == g["naive_reserved_gib"]
    assert round(100 * (1 - used / naive), 1) == g["naive_waste_pct"]
    assert round(paged * per_token / 2**30, 2) == g["paged_reserved_gib"]
    assert round(100 * (1 - used / paged), 1) == g["paged_waste_pct"]


def test_decode_growth_takes_one_block_per_boundary():
    # The allocator exercise: a per-step allocation without the boundary test
    # would hold one block per decode step; the right count is ceil(n / 16).
    pool = BlockPool(64, 16)
    t = pool.allocate(40)
    taken_at = []
    for cur in range(40, 140):
        b = pool.append_slot(t, cur)
        if b is not None:
            taken_at.append(cur)
    assert len(t) == math.ceil(140 / 16) == 9
    assert taken_at == [48, 64, 80, 96, 112, 128]
    assert pool.num_free() == 64 - 9


def test_pages_worked_counts():
    # A 40-token prompt takes 3 blocks (lesson 13.15, "How PagedAttention stores a request").
    assert BlockPool(8, 16).blocks_for(40) == 3
    # 1,500 shared prompt tokens fill 93 whole blocks (same lesson, its worked sizing example).
    assert 1500 // 16 == 93 and 93 * 16 == 1488


def _toy_loop(pool_blocks=12, block=16):
    """The lesson's practice loop, driven through the oracle pool: admit while
    a request's tokens fit, one token per running request per step with a new
    block when its last one is full, preempt the newest request when the pool
    is empty at that moment, release everything on finish."""
    pool = BlockPool(pool_blocks, block)
    waiting = [["A", 40, 40], ["B", 30, 24], ["C", 60, 30], ["D", 20, 16]]
    running = []  # [name, tokens, left, table]
    log, step = [], 0
    while waiting or running:
        while waiting and pool.can_allocate(waiting[0][1]):
            name, length, left = waiting.pop(0)
            table = pool.allocate(length)
            running.append([name, length, left, table])
            log.append(f"step {step:2d}: admit {name} with {length} tokens ({len(table)} blocks), "
                       f"free={pool.num_free()}")
        step += 1
        for r in list(running):
            if not any(r is x for x in running):
                continue
            needs_block = r[1] % block == 0
            if needs_block and pool.num_free() == 0:
                victim = running.pop()
                pool.release(victim[3])
                waiting.insert(0, [victim[0], victim[1], victim[2]])
                log.append(f"step {step:2d}: preempt {victim[0]} at {victim[1]} tokens, free={pool.num_free()}")
                if victim is r:
                    continue
            if needs_block:
                assert pool.append_slot(r[3], r[1]) is not None
            else:
                assert pool.append_slot(r[3], r[1]) is None
            r[1] += 1
            r[2] -= 1
            if r[2] == 0:
                running.remove(r)
                pool.release(r[3])
                log.append(f"step {step:2d}: finish {r[0]} at {r[1]} tokens, free={pool.num_free()}")
    log.append(f"all done at step {step}")
    return log, pool


def test_printed_toy_serving_loop():
    want = [l.rstrip("\n") for l in open(os.path.join(GOLDEN, "toy_block_pool_loop.txt"))
            if not l.startswith("#")]
    got, pool = _toy_loop()
    assert got == want
    assert pool.num_free() == 12 and not pool.refs


def test_copy_on_write():
    pool = BlockPool(8, 16)
    a = pool.allocate(40)
    b = list(a)
    pool.share(b)
    assert all(pool.ref_count(x) == 2 for x in a)
    copy = pool.make_writable(b, 2)
    assert copy is not None and copy[0] == a[2] and copy[1] == b[2] != a[2]
    assert pool.ref_count(a[2]) == 1 and pool.ref_count(b[2]) == 1
    assert pool.make_writable(b, 2) is None            # now private
    assert pool.make_writable(a, 2) is None            # the original's only holder
    pool.release(a)
    assert pool.ref_count(a[0]) == 1 and pool.ref_count(a[2]) == 0
    pool.release(b)
    assert pool.num_free() == 8 and not pool.refs


def test_errors_leave_the_pool_unchanged():
    pool = BlockPool(4, 16)
    t = pool.allocate(40)
    with pytest.raises(PoolError):
        pool.allocate(40)                               # 3 needed, 1 free
    assert pool.num_free() == 1
    unheld = pool.free[0]
    with pytest.raises(PoolError):
        pool.release([t[0], unheld])                    # the second id is not held
    assert pool.num_free() == 1 and all(pool.ref_count(x) == 1 for x in t)
    with pytest.raises(PoolError):
        BlockPool(3, 16, free_order=[0, 0, 1])


def test_prepare_step_hand_worked():
    # Prefill of request A's 40 tokens, and one decode token of request B at
    # position 52 (its 53rd token): slot = table[p // 16] * 16 + p % 16.
    slots, pos, rows, lens = prepare_step([[41, 9, 33], [41, 9, 37, 45]], [0, 52], [40, 1], 16, 5)
    assert slots[:16] == list(range(41 * 16, 41 * 16 + 16))
    assert slots[16:32] == list(range(9 * 16, 9 * 16 + 16))
    assert slots[32:40] == list(range(33 * 16, 33 * 16 + 8))
    assert slots[40:] == [45 * 16 + 4]
    assert pos == list(range(40)) + [52]
    assert rows == [[41, 9, 33, -1, -1], [41, 9, 37, 45, -1]]
    assert lens == [40, 53]
    with pytest.raises(PoolError):
        prepare_step([[1, 2]], [30], [3], 16, 4)        # position 32 needs a third block


def test_random_operations_keep_the_books():
    """Brute force: after any sequence of operations every block is either free
    or held, the counts equal the number of tables holding the block, and
    every table covers exactly its sequence's tokens."""
    rng = np.random.default_rng(3)
    pool = BlockPool(40, 16, free_order=rng.permutation(40))
    seqs = []  # [table, length]
    for _ in range(2000):
        op = rng.integers(0, 5)
        try:
            if op == 0:
                n = int(rng.integers(1, 70))
                seqs.append([pool.allocate(n), n])
            elif op == 1 and seqs:
                s = seqs[rng.integers(len(seqs))]
                pool.append_slot(s[0], s[1])
                s[1] += 1
            elif op == 2 and seqs:
                s = seqs[rng.integers(len(seqs))]
                pool.share(s[0])
                seqs.append([list(s[0]), s[1]])
            elif op == 3 and seqs:
                s = seqs.pop(rng.integers(len(seqs)))
                pool.release(s[0])
            elif op == 4 and seqs:
                s = seqs[rng.integers(len(seqs))]
                if s[0]:
                    pool.make_writable(s[0], int(rng.integers(len(s[0]))))
        except PoolError:
            pass
        held = {}
        for t, n in seqs:
            assert len(t) == math.ceil(n / 16)
            for b in t:
                held[b] = held.get(b, 0) + 1
        assert held == pool.refs
        assert sorted(pool.free + list(held)) == list(range(40))


def test_copy_on_write_keeps_every_reader_correct():
    """Through the pool and the block copy: after a writer's shared block is
    copied, both tables still read the same K/V at every position, blocks not
    named are untouched, and the writer can then change its copy without the
    reader seeing it."""
    rng = np.random.default_rng(5)
    pool = BlockPool(12, 16)
    kc = rng.standard_normal((12, 16, 2, 8))
    vc = rng.standard_normal((12, 16, 2, 8))
    a = pool.allocate(40)
    b = list(a)
    pool.share(b)
    copy = pool.make_writable(b, 2)
    k2, v2 = oracle.copy_blocks(kc, vc, [copy])
    for p in range(40):
        for t in (a, b):
            assert np.array_equal(k2[t[p // 16], p % 16], kc[a[p // 16], p % 16])
            assert np.array_equal(v2[t[p // 16], p % 16], vc[a[p // 16], p % 16])
    untouched = [i for i in range(12) if i != copy[1]]
    assert np.array_equal(k2[untouched], kc[untouched]) and np.array_equal(v2[untouched], vc[untouched])
    # The writer's new token lands in its private block only.
    k3, v3 = oracle.reshape_and_cache(np.ones((1, 2, 8)), np.ones((1, 2, 8)), k2, v2,
                                      np.array([b[40 // 16] * 16 + 40 % 16]))
    assert np.array_equal(k3[a[2], 8], k2[a[2], 8]) and (k3[b[2], 8] == 1).all()


def test_copy_blocks_skips_pairs_outside_the_pool():
    kc = np.arange(4 * 16 * 2, dtype=np.float64).reshape(4, 16, 2)
    vc = -kc
    k2, v2 = oracle.copy_blocks(kc, vc, [[0, 7], [-1, 2], [1, 3]])
    assert np.array_equal(k2[3], kc[1]) and np.array_equal(v2[3], vc[1])
    assert np.array_equal(k2[:3], kc[:3]) and np.array_equal(v2[:3], vc[:3])

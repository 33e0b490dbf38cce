"""Host block pool and block-table builder of libpda against the oracle's pool
model: identical tables, slots, free lists and reference counts (bit-exact),
plus the invariants of paged allocation (section 9.5 of "9 Decode and KV
Cache"; SoK paper section 2.5): no block handed out twice, all-or-nothing
allocation with ENOSPC as the preemption signal, copy-on-write for the block
that receives a row's newest token."""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth
import decode_attention_paged_slot_amd as pda

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_request_a_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "block_lookup.json")))["request_a"]
    order = [7, 2, 15] + [i for i in range(20) if i not in (7, 2, 15)]
    pool = pda.Pool(20, order)
    table, slots = pool.build_block_table([g["tokens"]], 16, 4)
    assert list(table[0]) == g["physical_blocks"] + [-1]
    assert slots[0] == oracle.slot_of(table[0], g["tokens"] - 1, 16)


def _same_state(p: pda.Pool, o: oracle.OraclePool):
    assert p.num_free() == o.num_free()
    for i in range(o.num_blocks):
        assert p.refcount(i) == o.ref[i]


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), B=st.integers(0, 9), shared=st.integers(0, 6),
       extra=st.integers(0, 20))
def test_builder_matches_oracle_pool(seed, B, shared, extra):
    r = np.random.default_rng(seed)
    ctx = r.integers(0, 200, size=B).astype(np.int32)
    need = int(synth.blocks_needed(ctx, 16).sum()) + shared
    nb = max(1, need + extra)
    order = synth.free_order(nb, r)
    p, o = pda.Pool(nb, order), oracle.OraclePool(nb, order)
    sp, so = p.alloc(shared), o.alloc(shared)
    assert list(sp) == list(so)
    mb = int(max(1, synth.blocks_needed(ctx, 16).max() if B else 1))
    t1, s1 = p.build_block_table(ctx, 16, mb, sp)
    t2, s2 = o.build_block_table(ctx, 16, mb, so)
    assert (t1 == t2).all() and (s1 == s2).all()
    _same_state(p, o)
    # every live entry maps to an allocated block; private blocks are unique
    live = t1[t1 >= 0]
    counts = np.bincount(live, minlength=nb)
    for i in range(nb):
        if i not in set(sp):
            assert counts[i] <= 1
    # newest token's block is private (refcount 1) and the slot points into it
    for b in range(B):
        if ctx[b] > 0:
            assert p.refcount(int(s1[b] // 16)) == 1
            assert s1[b] == oracle.slot_of(t1[b], int(ctx[b]) - 1, 16)
        else:
            assert s1[b] == -1
    # release everything in some order: both sides agree and the pool refills
    ids = list(live) + list(sp)
    r.shuffle(ids)
    p.free(ids)
    o.release(ids)
    _same_state(p, o)
    assert p.num_free() == nb


def test_enospc_is_all_or_nothing():
    p = pda.Pool(10)
    before = p.num_free()
    with pytest.raises(pda.NoSpace):
        p.build_block_table([64, 64, 64], 16, 4)      # needs 12 of 10
    assert p.num_free() == before
    with pytest.raises(pda.NoSpace):
        p.alloc(11)
    assert p.num_free() == before
    ids = p.alloc(10)
    assert sorted(ids) == list(range(10)) and p.num_free() == 0


def test_invalid_requests_change_nothing():
    p = pda.Pool(8)
    a = p.alloc(3)
    with pytest.raises(pda.PdaError):
        p.free([int(a[0]), int(a[0])])                # released twice, referenced once
    with pytest.raises(pda.PdaError):
        p.share([7])                                  # not allocated
    with pytest.raises(pda.PdaError):
        p.build_block_table([100], 16, 2)             # needs 7 blocks, table holds 2
    with pytest.raises(pda.PdaError):
        p.build_block_table([40], 16, 4, [7])         # shared id not allocated
    with pytest.raises(pda.PdaError):
        pda.Pool(4, [0, 1, 1, 3])                     # not a permutation
    assert p.num_free() == 5
    assert [p.refcount(int(i)) for i in a] == [1, 1, 1]


def test_copy_on_write_shared_prefix():
    p = pda.Pool(64, list(range(63, -1, -1)))
    prefix = p.alloc(4)
    table, slots = p.build_block_table([70, 64, 30, 5, 0], 16, 5, prefix)
    # 70 tokens: 5 blocks, first 4 shared; 64 tokens: 4 blocks, first 3 shared
    assert list(table[0, :4]) == list(prefix) and table[0, 4] not in prefix
    assert list(table[1, :3]) == list(prefix[:3]) and table[1, 3] not in prefix
    assert table[2, 0] == prefix[0] and table[2, 1] not in prefix
    assert table[3, 0] not in prefix                  # one block: always private
    assert (table[4] == -1).all() and slots[4] == -1
    refs = [p.refcount(int(i)) for i in prefix]
    assert refs == [1 + 3, 1 + 2, 1 + 2, 1 + 1]

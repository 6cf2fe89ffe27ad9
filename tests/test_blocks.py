"""Host block manager (reference counts, copy-on-write) and the oracle's
block copy, on the CPU."""
import numpy as np
import pytest

from oracle import ref
from workloads import blocks


def test_allocate_fork_append_release():
    bm = blocks.BlockManager(8)
    a = bm.allocate(0, 20)                     # 2 blocks, second one partial
    assert len(a) == 2 and all(bm.ref[b] == 1 for b in a)
    bm.fork(0, 1)
    assert all(bm.ref[b] == 2 for b in a)
    slot, copy = bm.append_slot(0)            # token 20 into a shared partial block
    assert copy is not None and copy[0] == a[1]
    new = copy[1]
    assert slot == new * 16 + 4 and bm.tables[0] == [a[0], new]
    assert bm.ref[a[1]] == 1 and bm.ref[new] == 1 and bm.ref[a[0]] == 2
    slot, copy = bm.append_slot(1)            # the old block is now private to 1
    assert copy is None and slot == a[1] * 16 + 4
    bm.check()
    for _ in range(12):                        # fill block 2 of seq 0 to 32 tokens
        bm.append_slot(0)
    assert bm.lens[0] == 33 and len(bm.tables[0]) == 3   # crossed into a fresh block
    bm.check()
    bm.release(1)
    assert bm.ref[a[1]] == 0 and a[1] in bm.free and bm.ref[a[0]] == 1
    bm.release(0)
    assert len(bm.free) == 8 and not bm.ref.any()


def test_full_shared_block_needs_no_copy():
    bm = blocks.BlockManager(6)
    bm.allocate(0, 32)
    bm.fork(0, 1)
    slot, copy = bm.append_slot(1)            # both blocks full: a fresh block, no copy
    assert copy is None and len(bm.tables[1]) == 3 and bm.tables[1][:2] == bm.tables[0]
    bm.check()


def test_out_of_blocks():
    bm = blocks.BlockManager(2)
    bm.allocate(0, 32)
    with pytest.raises(blocks.OutOfBlocks):
        bm.append_slot(0)


def test_scenario_invariants():
    sc = blocks.cow_scenario(3)
    n_copies = sum(len(s.pairs) for s in sc.steps)
    assert n_copies > 0
    for st in sc.steps:
        # copy destinations are fresh, distinct and never a source
        assert len(set(st.pairs[:, 1].tolist())) == len(st.pairs)
        assert not set(st.pairs[:, 1].tolist()) & set(st.pairs[:, 0].tolist())
        # slots: distinct, inside each sequence's last block
        assert len(set(st.slots.tolist())) == len(st.slots)
        for i in range(len(st.seqs)):
            L = int(st.context_lens[i])
            assert st.slots[i] == st.block_table[i, (L - 1) // 16] * 16 + (L - 1) % 16


def test_oracle_copy_blocks():
    rng = np.random.default_rng(2)
    kp = rng.standard_normal((6, 16, 2, 8)).astype(np.float16)
    vp = rng.standard_normal((6, 16, 2, 8)).astype(np.float16)
    ks = rng.random((6, 2, 16)).astype(np.float32)
    vs = rng.random((6, 2, 16)).astype(np.float32)
    pairs = np.array([[1, 4], [1, 5], [3, 0]], np.int32)
    k2, v2, ks2, vs2 = ref.ref_copy_blocks(kp, vp, pairs, ks, vs)
    for src, dst in pairs:
        for tkn in range(16):
            for g in range(2):
                for d in range(8):
                    assert k2[dst, tkn, g, d] == kp[src, tkn, g, d]
                    assert v2[dst, tkn, g, d] == vp[src, tkn, g, d]
                assert ks2[dst, g, tkn] == ks[src, g, tkn] and vs2[dst, g, tkn] == vs[src, g, tkn]
    untouched = [1, 2, 3]
    assert np.array_equal(k2[untouched], kp[untouched])
    with pytest.raises(ValueError):
        ref.ref_copy_blocks(kp, vp, np.array([[1, 4], [2, 4]]))      # repeated dst
    with pytest.raises(ValueError):
        ref.ref_copy_blocks(kp, vp, np.array([[1, 4], [4, 2]]))      # dst is also a src
    with pytest.raises(ValueError):
        ref.ref_copy_blocks(kp, vp, np.array([[1, 6]]))              # out of range

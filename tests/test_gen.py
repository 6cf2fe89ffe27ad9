"""Structure of the seeded synthetic workloads (host only)."""
import numpy as np
import pytest

from workloads import gen


def test_llama2_7b_table_is_85_percent_contiguous():
    wl = gen.make("llama2_7b", poison=False)
    assert wl.block_table.shape == (32, 256) and wl.num_blocks == 8192
    assert np.all(wl.context_lens == 4096)
    ident = np.arange(8192).reshape(32, 256)
    keep = (wl.block_table == ident).sum()
    assert keep == 8192 - 1229                       # 15 % deranged, none fixed
    assert sorted(wl.block_table.ravel().tolist()) == list(range(8192))


def test_long128k_table_and_sizes():
    wl = gen.make("long128k_int8", poison=False)
    assert wl.block_table.shape == (4, 8192) and wl.num_blocks == 32768
    assert np.all(wl.context_lens == 131072) and wl.partition_size == 512
    assert len(np.unique(wl.block_table)) == 32768
    assert gen.kv_ideal_bytes(wl) == 524288 * 8 * 264


def test_gqa70b_occupancy_and_shuffle():
    wl = gen.make("gqa70b_mixed")
    used = sum(gen.cdiv(int(L), 16) for L in wl.context_lens)
    assert abs(used / wl.num_blocks - 0.95) < 1e-3
    assert wl.context_lens.min() >= 128 and wl.context_lens.max() <= 8192
    ids = np.concatenate([wl.block_table[b, :gen.cdiv(int(L), 16)]
                          for b, L in enumerate(wl.context_lens)])
    assert len(np.unique(ids)) == len(ids) and ids.max() < wl.num_blocks


def test_prefix_shared_structure():
    wl = gen.make("prefix_shared")
    assert np.all(wl.block_table[:, :64] == wl.block_table[0, :64])
    assert np.all((wl.context_lens >= 1040) & (wl.context_lens <= 1536))
    priv = np.concatenate([wl.block_table[b, 64:gen.cdiv(int(L), 16)]
                           for b, L in enumerate(wl.context_lens)])
    assert len(np.unique(priv)) == len(priv)
    assert not set(priv.tolist()) & set(wl.block_table[0, :64].tolist())
    # twin: private copies hold the prefix's block data
    for b in range(wl.batch):
        assert np.array_equal(wl.twin_src[wl.twin_table[b, :64]], wl.block_table[b, :64])


def test_tiny_blocks_distinct_and_new_slots():
    wl = gen.make("tiny_gqa")
    ids = np.concatenate([wl.block_table[b, :gen.cdiv(int(L), 16)]
                          for b, L in enumerate(wl.context_lens)])
    assert len(np.unique(ids)) == len(ids)
    for b, L in enumerate(wl.context_lens):
        t = int(L) - 1
        assert wl.new_slots[b] == wl.block_table[b, t // 16] * 16 + t % 16


@pytest.mark.parametrize("name", gen.ORDER)
def test_poison_covers_unused_and_tails(name):
    wl = gen.make(name, small=True)
    v = gen.fill_numpy(wl, new_slot_poison=False)
    bad = gen.poison_mask(wl)
    if wl.kv_dtype == "fp16":
        assert np.all(np.isnan(v["k_pool"][bad])) and np.all(np.isnan(v["v_pool"][bad]))
        assert not np.isnan(v["k_pool"][~bad]).any()
    else:
        ks = v["k_scale"].transpose(0, 2, 1)
        assert np.all(np.isnan(ks[bad])) and not np.isnan(ks[~bad]).any()
    # determinism
    v2 = gen.fill_numpy(gen.make(name, small=True), new_slot_poison=False)
    assert np.array_equal(v["q"], v2["q"])

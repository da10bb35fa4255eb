"""The seeded input generators: reproducible, well-formed, poisoned where unused."""
import numpy as np

from workloads import (BLOCK_SIZE, config0, config1, config4, lens_config2, lens_config3,
                       make_prefill, permute_block_ids, unshare_blocks)


def _check_tables(tables, lens, nb):
    need = (lens.astype(np.int64) + 15) // 16
    for s in range(lens.shape[0]):
        row = tables[s]
        assert (row[:need[s]] >= 0).all() and (row[:need[s]] < nb).all()
        assert (row[need[s]:] == -1).all()


def test_config0_shape_and_reproducible():
    a, b = config0(), config0()
    assert a.decode.context_lens.tolist() == [1, 7, 16, 33]
    assert np.array_equal(a.decode.block_tables, b.decode.block_tables)
    assert a.k_host.tobytes() == b.k_host.tobytes()
    assert a.num_blocks == 16 and a.head_dim == 64 and a.dtype == "f32"
    assert a.scale == np.float32(1 / 8)
    _check_tables(a.decode.block_tables, a.decode.context_lens, 16)
    used = a.decode.block_tables[a.decode.block_tables >= 0]
    assert len(set(used.tolist())) == used.size == 6
    assert len(set(a.slot_mapping.tolist())) == 4


def test_config0_poison_and_newest_slot_hole():
    w = config0()
    ht = w.host_tables(w.decode.block_tables)
    for s, L in enumerate(w.decode.context_lens):
        last = (L - 1) // 16
        b = ht[s, last]
        rows = L - last * 16
        assert np.isnan(w.k_host[b, :, rows:, :]).all()
        assert np.isnan(w.k_host[b, :, rows - 1, :]).all()  # slot the scatter fills
        if rows > 1:
            assert np.isfinite(w.k_host[b, :, :rows - 1, :]).all()


def test_config1_ranges_unique_blocks():
    w = config1()
    g = w.decode
    assert g.num_seqs == 64 and w.num_heads == 32 and w.num_kv_heads == 32
    assert g.context_lens.min() >= 128 and g.context_lens.max() <= 2048
    _check_tables(g.block_tables, g.context_lens, w.num_blocks)
    used = g.block_tables[g.block_tables >= 0]
    assert len(set(used.tolist())) == used.size
    assert w.k_host.dtype == np.uint16


def test_config2_and_3_length_draws():
    rng = np.random.default_rng(0)
    l2 = lens_config2(rng, 10000)
    assert l2.min() >= 16 and l2.max() <= 4096
    assert abs(np.median(l2) - 1024) < 40
    l3 = lens_config3(rng, 1000)
    assert l3.min() >= 8192 and l3.max() <= 32768


def test_config4_sharing_structure():
    w = config4(num_prompts=4, samples=3, shared_prefix=64, max_private=40, num_prefill=2,
                chunk=32, max_prefix=48, num_blocks=128, heads=2, head_dim=16)
    t = w.decode.block_tables
    for p in range(4):
        rows = t[3 * p:3 * p + 3]
        assert (rows[:, :4] == rows[0, :4]).all()
    # private blocks are not shared
    priv = [int(x) for s in range(12) for x in t[s, 4:] if x >= 0]
    assert len(priv) == len(set(priv))
    pre = w.prefill
    assert np.diff(pre.query_start_loc).tolist() == [32, 32]
    assert (pre.context_lens >= 32).all()
    all_ids = set(int(x) for x in t.ravel() if x >= 0) | set(int(x) for x in pre.block_tables.ravel() if x >= 0)
    assert all_ids == set(w.host_ids.tolist())


def test_permutation_and_unsharing_keep_contents():
    w = config0()
    w2 = permute_block_ids(w, 3)
    ht1, ht2 = w.host_tables(w.decode.block_tables), w2.host_tables(w2.decode.block_tables)
    for s, L in enumerate(w.decode.context_lens):
        for j in range((L + 15) // 16):
            assert w.k_host[ht1[s, j]].tobytes() == w2.k_host[ht2[s, j]].tobytes()
    w = config4(num_prompts=2, samples=3, shared_prefix=32, max_private=20, num_prefill=1,
                chunk=16, max_prefix=16, num_blocks=64, heads=2, head_dim=16)
    w3 = unshare_blocks(w)
    t3 = w3.decode.block_tables
    used = [int(x) for x in t3.ravel() if x >= 0]
    assert len(used) == len(set(used))


def test_prefill_builder():
    w = make_prefill("p", 1, "bf16", [0, 20], [16, 5], 4, 2, 64, 16)
    g = w.prefill
    assert g.query.shape == (21, 4, 64)
    assert g.context_lens.tolist() == [16, 25]
    assert g.max_query_len == 16

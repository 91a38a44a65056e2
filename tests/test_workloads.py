"""The seeded generators: determinism and the structural invariants the paged layout relies on."""

import numpy as np
import pytest
import torch

from workloads import CONFIG_NAMES, algorithmic_bytes, build_structure, custom_structure, live_slot_mask, materialize


@pytest.mark.parametrize("name", CONFIG_NAMES)
def test_structure_invariants(name):
    st = build_structure(name)
    again = build_structure(name)
    np.testing.assert_array_equal(st.block_tables, again.block_tables)
    np.testing.assert_array_equal(st.context_lens, again.context_lens)
    B, mb, bs = st.num_seqs, st.max_blocks_per_seq, st.block_size
    assert st.block_tables.shape == (B, mb)
    assert st.context_lens.max() <= st.max_context_len <= mb * bs
    nblk = st.blocks_per_seq()
    shared = st.notes["shared_prefix_blocks"]
    private = []
    for s in range(B):
        live = st.block_tables[s, : nblk[s]]
        assert (live >= 0).all() and (live < st.poison_block).all()
        assert (st.block_tables[s, nblk[s]:] == st.poison_block).all()
        private.extend(live[shared:].tolist())
        L = int(st.context_lens[s])
        assert st.slot_mapping[s] == st.block_tables[s, (L - 1) // bs] * bs + (L - 1) % bs
    # private blocks (including copy-on-write destinations) are never reused
    assert len(private) == len(set(private))
    if shared:
        assert (st.block_tables_pre[:, :shared] == st.block_tables_pre[0, :shared]).all()
        assert set(st.copy_pairs[:, 0]) <= set(st.block_tables_pre[0, :shared].tolist())
        assert not set(st.copy_pairs[:, 1]) & set(st.block_tables_pre.ravel().tolist())


def test_configs_match_their_descriptions():
    c1 = build_structure("tiny_fp32")
    assert c1.context_lens.tolist() == [5, 17, 33, 64] and c1.num_blocks == 64 and c1.dtype == "f32"
    c2 = build_structure("llama2_7b")
    assert c2.num_seqs == 64 and c2.context_lens.min() >= 128 and c2.context_lens.max() <= 2048
    assert c2.num_blocks == int(np.ceil(1.1 * c2.blocks_per_seq().sum() - 1e-9)) + 1
    c3 = build_structure("mixed_len")
    lens = c3.context_lens
    assert ((lens >= 32) & (lens <= 500)).sum() == 179 and ((lens >= 1024) & (lens <= 4096)).sum() == 77
    free = 1 - c3.blocks_per_seq().sum() / (c3.num_blocks - 1)
    assert 0.19 < free < 0.21
    c4 = build_structure("mistral_gqa_prefix")
    assert c4.group_size == 4 and (c4.context_lens == 4096).all() and c4.copy_pairs.shape == (32, 2)
    assert (c4.block_tables[:32, 63] == c4.copy_pairs[:, 1]).all()
    c5 = build_structure("llama2_70b_gqa")
    assert c5.group_size == 8 and c5.block_size == 256 and c5.partition_size == 512
    b = algorithmic_bytes(c2)
    assert b["kv"] == int(c2.context_lens.astype(np.int64).sum()) * 32 * 128 * 2 * 2


def test_materialize_poisons_every_non_live_slot():
    st = custom_structure("t", 5, [5, 17, 33, 0], 4, 2, 16, 16, "bf16", pool_factor=1.5)
    for include in (True, False):
        t = materialize(st, "cpu", include_new_token=include)
        mask = live_slot_mask(st, include)
        nan = torch.isnan(t["key_cache"].float()).all(dim=-1).all(dim=-1).numpy()
        assert (nan == ~mask).all()
        assert not torch.isnan(t["value_cache"].float()[torch.from_numpy(mask)]).any()
        assert torch.isnan(t["value_cache"].float()[st.poison_block]).all()
    a = materialize(st, "cpu")
    b = materialize(st, "cpu")
    assert torch.equal(a["query"], b["query"]) and torch.equal(a["key_cache"].view(torch.int16),
                                                             b["key_cache"].view(torch.int16))


def test_rejects_inconsistent_requests():
    with pytest.raises(ValueError):
        custom_structure("t", 1, [5], 3, 2, 16, 16, "f32")
    with pytest.raises(ValueError):
        custom_structure("t", 1, [20], 2, 2, 16, 16, "f32", shared_prefix_blocks=2)
    with pytest.raises(ValueError):
        custom_structure("t", 1, [200], 2, 2, 16, 16, "f32", pool_blocks=5)

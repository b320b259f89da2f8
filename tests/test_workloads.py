"""Seeded input generators: determinism and the structure each workload promises."""
import torch

import workloads as W


def test_tiny_is_deterministic_and_shaped():
    a, b = W.make("tiny"), W.make("tiny")
    assert a.context_lens.tolist() == [1, 17, 32, 45]
    assert (a.num_q_heads, a.num_kv_heads, a.head_dim, a.num_blocks) == (4, 2, 64, 32)
    assert a.layers[0].k_cache.shape == (32, 16, 2, 64)
    assert a.layers[0].q.dtype == torch.float16 and a.scale == 1 / 8
    for x, y in ((a.layers[0].k_cache, b.layers[0].k_cache), (a.layers[0].q, b.layers[0].q),
                 (a.block_tables, b.block_tables)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    # 8 blocks used, distinct, taken from a permutation of the pool
    used = a.used_block_ids()
    assert len(used) == 8 and used.min() >= 0 and used.max() < 32


def test_slots_point_at_last_token():
    wl = W.make("tiny")
    for s, L in enumerate(wl.context_lens.tolist()):
        slot = int(wl.slot_mapping[s])
        assert slot // 16 == int(wl.block_tables[s, (L - 1) // 16]) and slot % 16 == (L - 1) % 16


def test_structure_of_named_configs():
    q = W.make("qwen3", values=False)
    assert q.num_seqs == 60 and q.context_lens.min() >= 64 and q.context_lens.max() <= 256
    t = W.make("tinyllama", values=False)
    assert t.num_seqs == 256 and 512 <= t.context_lens.min() and t.context_lens.max() <= 2048
    assert t.num_q_heads // t.num_kv_heads == 8 and t.head_dim == 64
    lg = W.make("llama7b_long", values=False)
    assert lg.context_lens.tolist() == [32768] * 32
    assert len(lg.used_block_ids()) == 1024 + 16 * 1024 + 16 * 2048
    for s in range(1, 16):
        assert torch.equal(lg.block_tables[s, :1024], lg.block_tables[0, :1024])
    assert not torch.equal(lg.block_tables[16, :1024], lg.block_tables[0, :1024])
    sk = W.make("skewed", values=False)
    lens = sk.context_lens
    assert sk.num_seqs == 512 and int(lens.max()) == 131072 and int((lens == 131072).sum()) == 1
    assert int((lens == 1).sum()) >= 64 and int(lens.min()) >= 1
    need = sum(-(-int(L) // 16) for L in lens)
    assert need <= sk.num_blocks and need / sk.num_blocks > 0.97
    # every sequence's blocks are distinct physical blocks (no accidental sharing)
    assert len(sk.used_block_ids()) == need


def test_poison_marks_only_unread_slots():
    wl = W.make("tiny")
    W.poison_unread(wl)
    k = wl.layers[0].k_cache.float()
    for s, L in enumerate(wl.context_lens.tolist()):
        n = -(-L // 16)
        rows = k[wl.block_tables[s, :n].long()].reshape(n * 16, 2, 64)
        assert torch.isfinite(rows[:L]).all()
        assert torch.isnan(rows[L:]).all()

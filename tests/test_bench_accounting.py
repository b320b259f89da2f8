"""The benchmark's byte accounting (the numerator of every GB/s figure and of
`roofline.achieved`) against an independent count: every token position a
decode call reads, walked through its block table to (physical block,
offset) pairs and made distinct with numpy, so that blocks shared by several
sequences (the Llama-7B shape's prefix cache) count once; plus q and out,
the table entries and lengths the call reads, and the fused cache write's new
rows (read once, stored once) and slots."""
import numpy as np
import pytest
import torch

import bench
import workloads as W


def independent_bytes(wl, fused):
    lens = wl.context_lens.numpy().astype(np.int64)
    tables = wl.block_tables.numpy().astype(np.int64)
    S, Hq, Hkv, D, e = wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, 2
    row = Hkv * D * e                                     # one token's K (or V) row, all heads
    flat = []
    for s, L in enumerate(lens):
        t = np.arange(L)
        flat.append(tables[s, t // 16] * 16 + t % 16)     # physical slot of every position read
    slots = np.concatenate(flat) if flat else np.zeros(0, np.int64)
    kv_unique = len(np.unique(slots)) * row * 2           # K and V
    kv_logical = int(lens.sum()) * row * 2
    q_out = 2 * S * Hq * D * e
    tables_read = int(((lens + 15) // 16).sum()) * 4 + S * 4
    write = (2 * S * row * 2 + S * 4) if wl.slot_mapping is not None else 0
    return kv_logical, kv_unique + q_out + tables_read + (write if fused else 0)


@pytest.mark.parametrize("name", ["tiny", "qwen3", "tinyllama", "llama7b_long", "skewed"])
@pytest.mark.parametrize("fused", [True, False])
def test_decode_bytes_match_an_independent_count(name, fused):
    wl = W.make(name, values=False)
    acc = bench.decode_bytes(torch, wl, fused)
    kv_logical, call = independent_bytes(wl, fused)
    assert acc["kv_logical"] == kv_logical
    assert acc["call_alg"] == call


def test_shared_prefix_is_counted_once():
    """The Llama-7B shape: 16 sequences share their first 16384 tokens, so
    the unique K/V bytes are the logical bytes less 15 copies of the prefix."""
    wl = W.make("llama7b_long", values=False)
    row2 = wl.num_kv_heads * wl.head_dim * 2 * 2
    acc = bench.decode_bytes(torch, wl, False)
    other = acc["decode_alg"] - (acc["kv_logical"] - 15 * 16384 * row2)
    lens = wl.context_lens.numpy()
    assert other == (2 * wl.num_seqs * wl.num_q_heads * wl.head_dim * 2
                     + int(((lens + 15) // 16).sum()) * 4 + wl.num_seqs * 4)


@pytest.mark.parametrize("name,n_new", [("qwen3", 5), ("tinyllama", 3), ("llama7b_long", 5)])
def test_multi_query_bytes_match_an_independent_count(name, n_new):
    wl = W.make(name, values=False)
    T = wl.num_seqs * n_new
    kv_logical, alg = bench.multi_query_bytes(torch, wl, T)
    kv_logical_ref, decode_call = independent_bytes(wl, fused=False)
    assert kv_logical == kv_logical_ref
    # the decode call's bytes with T query and output rows instead of S, plus
    # the S + 1 query offsets
    S, Hq, D = wl.num_seqs, wl.num_q_heads, wl.head_dim
    assert alg == decode_call - 2 * S * Hq * D * 2 + 2 * T * Hq * D * 2 + (S + 1) * 4


@pytest.mark.parametrize("S,L,Hq,D", [(1, 1, 1, 64), (3, 17, 2, 64), (2, 100, 4, 128)])
def test_prefill_flops_match_brute_force(S, L, Hq, D):
    pairs = sum(1 for t in range(L) for k in range(L) if k <= t)   # causal (query, key) pairs
    assert bench.prefill_flops(S, L, Hq, D) == S * Hq * pairs * D * 2 * 2

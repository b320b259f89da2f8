"""Seeded random configurations of every call on the GPU vs the fp64 oracle.

Each case draws its dtype, head_dim, GQA group, KV heads, batch, lengths
(empty, one-token, block-edge and ragged ones mixed), partition length and,
for decode, whether the cache write is fused (and, for the planned call,
where each new row goes), from a seed of its own; all
inputs are valid. Tolerance as elsewhere: max |gpu - oracle| <= 2e-3 (fp16)
/ 1.5e-2 (bf16); pools after a write are compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_206_amd as mvk
import workloads as W
from gpu_helpers import TOL, bits, max_err, oracle_decode_all

pytestmark = pytest.mark.gpu

EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65]


def draw_shape(rng):
    dtype = str(rng.choice(["f16", "bf16"]))
    d = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4]))
    return dtype, d, g, hkv


def draw_lens(rng, n, hi, lo=0):
    lens = []
    for _ in range(n):
        r = rng.random()
        if r < 0.3:
            lens.append(max(lo, int(rng.choice(EDGE_LENS))))
        elif r < 0.4:
            lens.append(max(lo, int(16 * rng.integers(1, hi // 16 + 1))))   # whole blocks
        else:
            lens.append(int(rng.integers(max(lo, 1), hi + 1)))
    return lens


@pytest.mark.parametrize("case", range(16))
def test_random_decode(case):
    rng = np.random.default_rng(1000 + case)
    dtype, d, g, hkv = draw_shape(rng)
    lens = draw_lens(rng, int(rng.integers(1, 25)), int(rng.choice([80, 700, 2500])))
    p = int(rng.choice([0, 16, 32, 64, 256, 1024]))
    fused = bool(rng.random() < 0.5)
    nb = sum(-(-L // 16) for L in lens) + int(rng.integers(1, 8))
    wl = W.make_custom("r", dtype, lens, g * hkv, hkv, d, nb, 2000 + case)
    print(f"case {case}: {dtype} d={d} g={g} hkv={hkv} S={len(lens)} max L={max(lens)} "
          f"p={p} fused={fused}", flush=True)
    layer = wl.layers[0]
    kc, vc = bits(layer.k_cache), bits(layer.v_cache)
    slots = wl.slot_mapping.numpy()
    kc_ref, vc_ref = oracle.cache_write(kc, vc, bits(layer.key), bits(layer.value), slots)
    ref = oracle.paged_decode(bits(layer.q), kc_ref, vc_ref, wl.block_tables.numpy(),
                              wl.context_lens.numpy(), wl.scale, dtype)
    gw = wl.to("cuda")
    gl = gw.layers[0]
    if fused:
        out = mvk.paged_attention_decode(gl.q, gl.k_cache, gl.v_cache, gw.block_tables,
                                         gw.context_lens, gw.scale, max_context_len=max(lens),
                                         partition_tokens=p, new_key=gl.key, new_value=gl.value,
                                         slot_mapping=gw.slot_mapping)
    else:
        mvk.reshape_and_cache(gl.key, gl.value, gl.k_cache, gl.v_cache, gw.slot_mapping)
        out = mvk.paged_attention_decode(gl.q, gl.k_cache, gl.v_cache, gw.block_tables,
                                         gw.context_lens, gw.scale, max_context_len=max(lens),
                                         partition_tokens=p)
    torch.cuda.synchronize()
    assert max_err(out, ref, dtype) <= TOL[dtype]
    assert np.array_equal(bits(gl.k_cache), kc_ref)
    assert np.array_equal(bits(gl.v_cache), vc_ref)


@pytest.mark.parametrize("case", range(16))
def test_random_planned_decode(case):
    """The planned call (a plan, then the layer's call) on random batches
    within its scope: up to 300 sequences, contexts up to 7000 tokens (items
    needing several descriptors of blocks), and with the fused write new rows
    mostly at the newest position, some at an earlier position of the
    sequence's own context, in a block nobody reads, or nowhere (-1)."""
    rng = np.random.default_rng(5000 + case)
    dtype, d, g, hkv = draw_shape(rng)
    n = int(rng.integers(1, 31)) if rng.random() < 0.7 else int(rng.integers(200, 301))
    lens = draw_lens(rng, n, [80, 700, 2500, 7000][case % 4])
    fused = bool(rng.random() < 0.6)
    free = int(rng.integers(2, 9))
    nb = sum(-(-L // 16) for L in lens) + free
    wl = W.make_custom("r", dtype, lens, g * hkv, hkv, d, nb, 6000 + case)
    maxlen = max(lens)
    assert mvk.plan_size(len(lens), g * hkv, hkv, d, maxlen) is not None
    slots = wl.slot_mapping.clone()
    if fused:
        used = set(int(x) for x in wl.used_block_ids())
        free_rows = [b * 16 + r for b in range(nb) if b not in used for r in range(16)]
        rng.shuffle(free_rows)
        for s_ in range(len(lens)):
            r = rng.random()
            L = lens[s_]
            if r < 0.12 and L >= 2:              # an earlier token of its own context
                t = int(rng.integers(0, L - 1))
                slots[s_] = int(wl.block_tables[s_, t // 16]) * 16 + t % 16
            elif r < 0.2 and free_rows:           # a block nobody reads
                slots[s_] = free_rows.pop()
            elif r < 0.27:
                slots[s_] = -1
    print(f"case {case}: {dtype} d={d} g={g} hkv={hkv} S={len(lens)} max L={maxlen} "
          f"fused={fused}", flush=True)
    layer = wl.layers[0]
    kc, vc = bits(layer.k_cache), bits(layer.v_cache)
    if fused:
        kc, vc = oracle.cache_write(kc, vc, bits(layer.key), bits(layer.value), slots.numpy())
    ref = oracle_decode_all(bits(layer.q), kc, vc, wl.block_tables.numpy(),
                            wl.context_lens.numpy(), wl.scale, dtype)
    gw = wl.to("cuda")
    gl = gw.layers[0]
    sm = slots.cuda()
    plan = mvk.make_plan(gw.block_tables, gw.context_lens, g * hkv, hkv, d, maxlen,
                         slot_mapping=sm if fused else None)
    extra = dict(new_key=gl.key, new_value=gl.value) if fused else {}
    out = mvk.paged_attention_decode_planned(gl.q, gl.k_cache, gl.v_cache, plan, gw.scale,
                                             maxlen, **extra)
    torch.cuda.synchronize()
    assert max_err(out, ref, dtype) <= TOL[dtype]
    assert np.array_equal(bits(gl.k_cache), kc)
    assert np.array_equal(bits(gl.v_cache), vc)


@pytest.mark.parametrize("case", range(12))
def test_random_multi_query(case):
    rng = np.random.default_rng(3000 + case)
    dtype, d, g, hkv = draw_shape(rng)
    lens = draw_lens(rng, int(rng.integers(1, 13)), int(rng.choice([100, 900, 2000])), lo=1)
    news = [int(rng.integers(0, min(L, 40) + 1)) for L in lens]
    news[0] = max(news[0], 1)   # a call takes at least one query token
    p = int(rng.choice([0, 16, 64, 256]))
    nb = sum(-(-L // 16) for L in lens) + 3
    wl = W.make_custom("r", dtype, lens, g * hkv, hkv, d, nb, 4000 + case)
    q, qs = W.make_queries(wl, news, 5000 + case)
    print(f"case {case}: {dtype} d={d} g={g} hkv={hkv} lens={lens} news={news} p={p}",
          flush=True)
    layer = wl.layers[0]
    ref = oracle.paged_multi_query(bits(q), bits(layer.k_cache), bits(layer.v_cache),
                                   wl.block_tables.numpy(), wl.context_lens.numpy(), qs.numpy(),
                                   wl.scale, dtype)
    gw = wl.to("cuda")
    out = mvk.paged_attention_multi_query(q.to("cuda"), gw.layers[0].k_cache,
                                          gw.layers[0].v_cache, gw.block_tables, gw.context_lens,
                                          qs.to("cuda"), gw.scale, max_query_len=max(news),
                                          max_context_len=max(lens), partition_tokens=p)
    torch.cuda.synchronize()
    assert max_err(out, ref, dtype) <= TOL[dtype]


@pytest.mark.parametrize("case", range(12))
def test_random_planned_multi_query(case):
    """The multi-query call through a step's plan: shapes in its scope (not
    head_dim 128 with g = 1), up to 16 rows per item, contexts up to 7000
    tokens (short and long descriptors, items over several waves)."""
    rng = np.random.default_rng(8000 + case)
    dtype, d, g, hkv = draw_shape(rng)
    if d == 128 and g == 1:
        d = 64
    lens = draw_lens(rng, int(rng.integers(1, 40)), int(rng.choice([120, 900, 7000])), lo=1)
    news = [int(rng.integers(0, min(L, 16 // g) + 1)) for L in lens]
    news[0] = max(news[0], 1)
    nb = sum(-(-L // 16) for L in lens) + 3
    wl = W.make_custom("r", dtype, lens, g * hkv, hkv, d, nb, 9000 + case)
    q, qs = W.make_queries(wl, news, 9500 + case)
    print(f"case {case}: {dtype} d={d} g={g} hkv={hkv} lens={lens} news={news}", flush=True)
    layer = wl.layers[0]
    ref = oracle.paged_multi_query(bits(q), bits(layer.k_cache), bits(layer.v_cache),
                                   wl.block_tables.numpy(), wl.context_lens.numpy(), qs.numpy(),
                                   wl.scale, dtype)
    gw = wl.to("cuda")
    plan = mvk.make_plan(gw.block_tables, gw.context_lens, g * hkv, hkv, d, max(lens))
    out = mvk.paged_attention_multi_query_planned(q.to("cuda"), gw.layers[0].k_cache,
                                                  gw.layers[0].v_cache, plan, qs.to("cuda"),
                                                  len(lens), gw.scale, max(news), max(lens))
    torch.cuda.synchronize()
    assert max_err(out, ref, dtype) <= TOL[dtype]


@pytest.mark.parametrize("case", range(10))
def test_random_prefill(case):
    rng = np.random.default_rng(6000 + case)
    dtype, d, g, hkv = draw_shape(rng)
    lens = draw_lens(rng, int(rng.integers(1, 9)), int(rng.choice([70, 300, 700])))
    write = bool(rng.random() < 0.7)
    pf = W.make_prefill(dtype, lens, g * hkv, hkv, d, seed=7000 + case,
                        extra_blocks=int(rng.integers(0, 5)))
    print(f"case {case}: {dtype} d={d} g={g} hkv={hkv} lens={lens} write={write}", flush=True)
    ref = oracle.prefill_attention(bits(pf.q), bits(pf.key), bits(pf.value), pf.cu_seqlens.numpy(),
                                   pf.scale, dtype)
    kc_ref, vc_ref = oracle.cache_write(bits(pf.k_cache), bits(pf.v_cache), bits(pf.key),
                                        bits(pf.value), pf.slot_mapping.numpy())
    gp = pf.to("cuda")
    kw = dict(k_cache=gp.k_cache, v_cache=gp.v_cache, slot_mapping=gp.slot_mapping) if write else {}
    out = mvk.prefill_attention(gp.q, gp.key, gp.value, gp.cu_seqlens, gp.scale,
                                max_seqlen=max(lens), **kw)
    torch.cuda.synchronize()
    if pf.q.shape[0]:
        assert max_err(out, ref, dtype) <= TOL[dtype]
    if write:
        assert np.array_equal(bits(gp.k_cache), kc_ref)
        assert np.array_equal(bits(gp.v_cache), vc_ref)

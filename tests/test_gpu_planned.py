"""Planned decode (a plan built once per step, read by every layer's call)
against the fp64 oracle: a dtype x head_dim x group sweep with empty,
one-token, block-edge and ragged contexts; every row written exactly once
for batches of 1..257 sequences with ties; fused cache write bit-exact;
determinism; NaN in every unread slot; the plan as a snapshot of the arrays
it was built from; several layers through one plan; a captured graph of the
plan and the layers' calls; and the full Qwen3- and TinyLlama-shaped steps."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_206_amd as mvk
import workloads as W
from gpu_helpers import TOL, bits, max_err, oracle_decode_all

pytestmark = pytest.mark.gpu


def oracle_step(wl, layer_idx, fused):
    """Oracle output of one layer (after the layer's cache write when fused)
    and the pools the write leaves."""
    l = wl.layers[layer_idx]
    kc, vc = bits(l.k_cache), bits(l.v_cache)
    if fused:
        kc, vc = oracle.cache_write(kc, vc, bits(l.key), bits(l.value), wl.slot_mapping.numpy())
    ref = oracle_decode_all(bits(l.q), kc, vc, wl.block_tables.numpy(), wl.context_lens.numpy(),
                            wl.scale, wl.dtype)
    return ref, kc, vc


def run_planned(g, layer_idx, fused, plan=None, out=None, maxlen=None):
    """The planned call on a workload already on the GPU (`maxlen`: the
    plan's host-side bound; read from the lengths when not given)."""
    l = g.layers[layer_idx]
    if maxlen is None:
        maxlen = int(g.context_lens.max().item())
    if plan is None:
        plan = mvk.make_plan(g.block_tables, g.context_lens, g.num_q_heads, g.num_kv_heads,
                             g.head_dim, maxlen, slot_mapping=g.slot_mapping if fused else None)
    if out is None:
        out = torch.full_like(l.q, float("nan"))
    extra = dict(new_key=l.key, new_value=l.value) if fused else {}
    mvk.paged_attention_decode_planned(l.q, l.k_cache, l.v_cache, plan, g.scale, maxlen, out=out,
                                       **extra)
    return out, plan


def check_layer(wl, layer_idx=0, fused=False, label=""):
    ref, kc, vc = oracle_step(wl, layer_idx, fused)
    g = wl.to("cuda")
    out, _ = run_planned(g, layer_idx, fused)
    torch.cuda.synchronize()
    err = max_err(out, ref, wl.dtype)
    print(f"planned {label} fused={fused}: {wl.num_seqs} seqs, max abs err {err:.3e}", flush=True)
    assert err <= TOL[wl.dtype], label
    if fused:
        assert np.array_equal(bits(g.layers[layer_idx].k_cache), kc)
        assert np.array_equal(bits(g.layers[layer_idx].v_cache), vc)
    return g, out


MIXED = [0, 1, 15, 16, 17, 31, 32, 33, 100, 255, 256, 257, 640, 1, 0, 48]


@pytest.mark.parametrize("fused", [False, True], ids=["plain", "fused_write"])
@pytest.mark.parametrize("dtype,D,hq,hkv", [
    ("f16", 64, 4, 4), ("bf16", 128, 8, 8),          # g = 1 (VALU policy)
    ("bf16", 128, 16, 8), ("f16", 64, 8, 4),          # g = 2
    ("f16", 128, 16, 4), ("bf16", 64, 32, 8),         # g = 4
    ("f16", 64, 32, 4), ("bf16", 128, 64, 8),         # g = 8
    ("bf16", 128, 8, 1), ("f16", 64, 6, 3),           # one KV head; three (item -> sequence division)
])
def test_planned_sweep(dtype, D, hq, hkv, fused):
    lens = [L if L > 0 else (0 if not fused else 1) for L in MIXED]
    wl = W.make_custom("p", dtype, lens, hq, hkv, D, sum(-(-L // 16) for L in lens) + 5,
                       100 + hq + D)
    check_layer(wl, 0, fused, f"{dtype} D={D} g={hq // hkv}")


@pytest.mark.parametrize("num_seqs", [1, 2, 7, 60, 129, 256, 257])
def test_planned_writes_every_row_once(num_seqs):
    """Ties, empty and one-token contexts, more items than bins and fewer:
    every output row is written (the output starts as NaN) and matches."""
    gen = torch.Generator().manual_seed(num_seqs)
    lens = torch.randint(0, 300, (num_seqs,), generator=gen)
    lens[::5] = 64                                   # ties
    lens[1::11] = 0
    lens[2::13] = 1
    wl = W.make_custom("p", "bf16", lens.tolist(), 16, 8, 128,
                       int(((lens + 15) // 16).sum()) + 3, 300 + num_seqs, new_rows=False)
    check_layer(wl, 0, False, f"{num_seqs} seqs")


@pytest.mark.parametrize("fused", [False, True], ids=["plain", "fused_write"])
def test_planned_short_descriptors_at_capacity(fused):
    """Short (32-int) descriptors at their limit: 258 sequences fill every
    bin with eight one-wave items, and contexts of 384, 383 and 369 tokens
    put 24 blocks (the short form's capacity) in one descriptor."""
    lens = [384, 383, 369, 1, 17, 200] * 43
    wl = W.make_custom("p", "bf16", lens, 16, 8, 128, sum(-(-L // 16) for L in lens) + 3, 77)
    assert mvk.plan_size(wl.num_seqs, 16, 8, 128, wl.max_context_len) == 258 * 8 * 32 * 4
    check_layer(wl, 0, fused, "short descriptors at capacity")


@pytest.mark.parametrize("fused", [False, True], ids=["plain", "fused_write"])
def test_planned_at_the_ranking_capacity(fused):
    """1024 sequences, the most one plan ranks (every workgroup holds all
    their keys in LDS), with ties, one-token contexts and longer ones."""
    gen = torch.Generator().manual_seed(1024)
    lens = torch.randint(1, 97, (1024,), generator=gen)
    lens[::7] = 48                                   # ties
    lens[3::17] = 1
    lens[5::101] = 700
    wl = W.make_custom("p", "f16", lens.tolist(), 8, 2, 64, int(((lens + 15) // 16).sum()) + 3,
                       1024)
    assert mvk.plan_size(1024, 8, 2, 64, wl.max_context_len) is not None
    assert mvk.plan_size(1025, 8, 2, 64, wl.max_context_len) is None
    check_layer(wl, 0, fused, "1024 sequences")


def test_planned_at_the_kv_head_capacity():
    """256 KV heads (the most a plan takes), g = 1 and g = 2: item i's head
    is i mod 256 through the multiply-high division."""
    for hq, D, dtype in ((256, 64, "bf16"), (512, 128, "f16")):
        lens = [1, 40, 333, 16, 17]
        wl = W.make_custom("p", dtype, lens, hq, 256, D, sum(-(-L // 16) for L in lens) + 2,
                           hq + D)
        assert mvk.plan_size(len(lens), hq, 256, D, wl.max_context_len) is not None
        assert mvk.plan_size(len(lens), 2 * 257, 257, D, wl.max_context_len) is None
        check_layer(wl, 0, True, f"256 KV heads, g = {hq // 256}")


@pytest.mark.parametrize("dtype,D,hq,hkv", [("bf16", 128, 8, 8), ("f16", 64, 32, 4)])
def test_planned_items_longer_than_one_descriptor(dtype, D, hq, hkv):
    """Contexts past 56 blocks (one wave descriptor) up to the planned path's
    7168 tokens: an item takes several waves, fewer items share a bin."""
    lens = [7168, 896, 897, 2600, 1, 17, 3000, 5000, 0, 911]
    wl = W.make_custom("p", dtype, lens, hq, hkv, D, sum(-(-L // 16) for L in lens) + 2,
                       600 + D, new_rows=False)
    check_layer(wl, 0, False, f"long items {dtype} D={D} g={hq // hkv}")


def planned_fused(wl, slots):
    """Planned call with the fused write at `slots` on fresh GPU copies:
    (out, k pool bits, v pool bits)."""
    g = wl.to("cuda")
    l = g.layers[0]
    sm = slots.cuda()
    maxlen = wl.max_context_len
    plan = mvk.make_plan(g.block_tables, g.context_lens, wl.num_q_heads, wl.num_kv_heads,
                         wl.head_dim, maxlen, slot_mapping=sm)
    out = mvk.paged_attention_decode_planned(l.q, l.k_cache, l.v_cache, plan, wl.scale, maxlen,
                                             new_key=l.key, new_value=l.value)
    torch.cuda.synchronize()
    return out, bits(l.k_cache), bits(l.v_cache)


def check_planned_fused(wl, slots, label):
    """Against the oracle's write-then-decode: pools bit-exact, output within
    the bar, bits repeatable."""
    layer = wl.layers[0]
    ek, ev = oracle.cache_write(bits(layer.k_cache), bits(layer.v_cache), bits(layer.key),
                                bits(layer.value), slots.numpy())
    ref = oracle_decode_all(bits(layer.q), ek, ev, wl.block_tables.numpy(),
                            wl.context_lens.numpy(), wl.scale, wl.dtype)
    out, k, v = planned_fused(wl, slots)
    assert np.array_equal(k, ek) and np.array_equal(v, ev), "fused store is not bit-exact"
    err = max_err(out, ref, wl.dtype)
    print(f"planned fused {label}: max abs err {err:.3e}", flush=True)
    assert err <= TOL[wl.dtype], label
    out2, _, _ = planned_fused(wl, slots)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def poison_slots(wl, slots):
    """NaN in the rows the cache write is about to replace: the call must
    not read their old bits."""
    nan = W.NAN_BITS[wl.dtype]
    for pool in (wl.layers[0].k_cache, wl.layers[0].v_cache):
        raw = pool.view(torch.int16).view(-1, wl.num_kv_heads * wl.head_dim)
        for sl in slots.tolist():
            if sl >= 0:
                raw[sl] = nan


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_planned_fused_newest_token(dtype, d, g):
    """The decode step's own token (the slot of position L-1): appended after
    the blocks, including contexts where it is alone in its block (L = 17,
    33) and the one-token context (the output is the new V row)."""
    lens = [1, 16, 17, 100, 255, 33, 2, 640]
    nb = sum(-(-L // 16) for L in lens) + 5
    wl = W.make_custom("pf", dtype, lens, 2 * g, 2, d, nb, seed=70 + g)
    W.poison_unread(wl)
    poison_slots(wl, wl.slot_mapping)
    check_planned_fused(wl, wl.slot_mapping, f"newest {dtype} D={d} g={g}")


@pytest.mark.parametrize("g", [1, 2, 4])
def test_planned_fused_other_slots(g):
    """Slots at an early position of the sequence's own context and at the
    first row of its last block (stored first by the wave that reads that
    block), in a block nobody reads, and negative (no write)."""
    lens = [40, 70, 5, 130, 16, 900]
    nb = sum(-(-L // 16) for L in lens) + 3
    wl = W.make_custom("pf", "bf16", lens, 2 * g, 2, 128, nb, seed=80 + g)
    bt = wl.block_tables
    used = set(int(x) for x in wl.used_block_ids())
    free_blk = next(b for b in range(nb) if b not in used)
    slots = wl.slot_mapping.clone()
    slots[0] = int(bt[0, 0]) * 16 + 3            # an early token of its own context
    slots[1] = int(bt[1, 4]) * 16 + 0            # first row of its last block
    slots[2] = free_blk * 16 + 7                 # a block nobody reads
    slots[3] = -1                                # no write this step
    slots[5] = int(bt[5, 20]) * 16 + 9           # a middle block of a many-wave item
    poison_slots(wl, slots)
    check_planned_fused(wl, slots, f"other slots g={g}")


def test_planned_is_deterministic_and_poison_proof():
    lens = [5, 300, 17, 129, 64, 1, 250, 33]
    wl = W.make_custom("p", "f16", lens, 16, 4, 64, 60, 400)
    W.poison_unread(wl)
    g, out1 = check_layer(wl, 0, False, "poisoned")
    out2, _ = run_planned(g, 0, False)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_planned_close_to_unplanned():
    """Both orders of summation are within the bound of the exact result."""
    wl = W.make("qwen3", layers=1)
    ref, _, _ = oracle_step(wl, 0, True)
    g = wl.to("cuda")
    l = g.layers[0]
    k0, v0 = l.k_cache.clone(), l.v_cache.clone()
    planned, _ = run_planned(g, 0, True)
    l.k_cache.copy_(k0)
    l.v_cache.copy_(v0)
    plain = mvk.paged_attention_decode(l.q, l.k_cache, l.v_cache, g.block_tables, g.context_lens,
                                       g.scale, max_context_len=wl.max_context_len,
                                       new_key=l.key, new_value=l.value,
                                       slot_mapping=g.slot_mapping)
    torch.cuda.synchronize()
    assert max_err(planned, ref, "bf16") <= TOL["bf16"]
    assert max_err(plain, ref, "bf16") <= TOL["bf16"]


def test_plan_is_a_snapshot_and_serves_every_layer():
    """One plan, three layers; the tables and lengths are overwritten after
    the plan is built, and the planned calls still read the plan's copy."""
    lens = [40, 200, 3, 96, 150]
    wl = W.make_custom("p", "bf16", lens, 16, 8, 128, 40, 500, layers=3)
    refs = [oracle_step(wl, i, True) for i in range(3)]
    g = wl.to("cuda")
    maxlen = wl.max_context_len
    plan = mvk.make_plan(g.block_tables, g.context_lens, 16, 8, 128, maxlen,
                         slot_mapping=g.slot_mapping)
    g.block_tables.fill_(-1)
    g.context_lens.zero_()
    g.slot_mapping.fill_(-1)
    for i in range(3):
        out, _ = run_planned(g, i, True, plan=plan, maxlen=maxlen)
        torch.cuda.synchronize()
        ref, kc, vc = refs[i]
        assert max_err(out, ref, "bf16") <= TOL["bf16"], i
        assert np.array_equal(bits(g.layers[i].k_cache), kc)


def test_planned_step_in_a_graph():
    """The plan and the layers' planned calls captured once; every replay
    (after unrelated eager work and a sync) matches the oracle and the eager
    bits."""
    wl = W.make("qwen3", layers=3)
    refs = [oracle_step(wl, i, True) for i in range(3)]
    g = wl.to("cuda")
    maxlen = wl.max_context_len
    plan = torch.empty(mvk.plan_size(60, 16, 8, 128, maxlen), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(l.q) for l in g.layers]

    def step():
        mvk.make_plan(g.block_tables, g.context_lens, 16, 8, 128, maxlen,
                      slot_mapping=g.slot_mapping, plan=plan)
        for i in range(3):
            run_planned(g, i, True, plan=plan, out=outs[i], maxlen=maxlen)
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(outs[i].view(torch.int16), eager[i].view(torch.int16)), (rep, i)
            assert max_err(outs[i], refs[i][0], "bf16") <= TOL["bf16"], (rep, i)
            assert np.array_equal(bits(g.layers[i].k_cache), refs[i][1])


@pytest.mark.parametrize("name", ["qwen3", "tinyllama"])
def test_planned_full_step_every_row(name):
    """The benchmark's planned step: one plan, then every layer's fused call;
    every row of every layer against the oracle, pools bit-exact."""
    wl = W.make(name, value_device="cuda")
    maxlen = wl.max_context_len
    host = [(bits(l.q), bits(l.k_cache), bits(l.v_cache), bits(l.key), bits(l.value))
            for l in wl.layers]
    bt, cl, sm = wl.block_tables.cuda(), wl.context_lens.cuda(), wl.slot_mapping.cuda()
    plan = mvk.make_plan(bt, cl, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, maxlen,
                         slot_mapping=sm)
    outs = []
    for l in wl.layers:
        outs.append(mvk.paged_attention_decode_planned(l.q, l.k_cache, l.v_cache, plan, wl.scale,
                                                       maxlen, new_key=l.key, new_value=l.value))
    torch.cuda.synchronize()
    worst = 0.0
    for i, (q, kc, vc, key, value) in enumerate(host):
        kc, vc = oracle.cache_write(kc, vc, key, value, wl.slot_mapping.numpy())
        assert np.array_equal(bits(wl.layers[i].k_cache), kc)
        assert np.array_equal(bits(wl.layers[i].v_cache), vc)
        ref = oracle_decode_all(q, kc, vc, wl.block_tables.numpy(), wl.context_lens.numpy(),
                                wl.scale, wl.dtype)
        err = max_err(outs[i], ref, wl.dtype)
        worst = max(worst, err)
        assert err <= TOL[wl.dtype], (name, i, err)
    print(f"planned {name}: {len(host)} layers x {wl.num_seqs} seqs, max abs err {worst:.3e}",
          flush=True)

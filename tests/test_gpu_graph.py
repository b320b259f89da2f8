"""Captured HIP graphs of the decode step (cache write + decode per layer),
of multi-query calls and of a prefill call: every replay is preceded by eager
work and a synchronisation, and every replayed output is checked against the
fp64 oracle at the parity tolerance (the pools bit for bit against the
oracle's cache write) as well as bit for bit against the eager result."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_206_amd as mvk
import workloads as W
from gpu_helpers import TOL, bits, max_err

pytestmark = pytest.mark.gpu


def run_step(wl, bt, cl, slots, outs, partition_tokens, ws, maxlen, fused=False):
    for l, out in zip(wl.layers, outs):
        if fused:
            mvk.paged_attention_decode(l.q, l.k_cache, l.v_cache, bt, cl, wl.scale,
                                       max_context_len=maxlen, out=out,
                                       partition_tokens=partition_tokens, workspace=ws,
                                       new_key=l.key, new_value=l.value, slot_mapping=slots)
            continue
        mvk.reshape_and_cache(l.key, l.value, l.k_cache, l.v_cache, slots)
        mvk.paged_attention_decode(l.q, l.k_cache, l.v_cache, bt, cl, wl.scale,
                                   max_context_len=maxlen, out=out,
                                   partition_tokens=partition_tokens, workspace=ws)


@pytest.mark.parametrize("fused", [False, True], ids=["separate_write", "fused_write"])
@pytest.mark.parametrize("case", ["single_pass", "split_merge", "work_list"])
def test_graph_replay_matches_eager(case, fused):
    if case == "single_pass":
        wl = W.make("qwen3", layers=3)
        p = 0
    elif case == "split_merge":
        wl = W.make_custom("g", "bf16", [900, 17, 1, 2000, 640], 32, 8, 128, 400, 21, layers=2)
        p = 256
    else:
        gen = torch.Generator().manual_seed(5)
        lens = torch.randint(1, 400, (200,), generator=gen).tolist()
        wl = W.make_custom("g", "f16", lens, 16, 8, 64, sum(-(-L // 16) for L in lens) + 8, 22,
                           layers=2)
        p = 32
    maxlen = wl.max_context_len          # host-side, before anything is captured
    # oracle: each layer's cache write, then decode over the written pools
    refs, pools = [], []
    for l in wl.layers:
        kc, vc = oracle.cache_write(bits(l.k_cache), bits(l.v_cache), bits(l.key), bits(l.value),
                                    wl.slot_mapping.numpy())
        pools.append((kc, vc))
        refs.append(oracle.paged_decode(bits(l.q), kc, vc, wl.block_tables.numpy(),
                                        wl.context_lens.numpy(), wl.scale, wl.dtype))
    wl = wl.to("cuda")
    bt, cl, slots = wl.block_tables, wl.context_lens, wl.slot_mapping
    nbytes, _ = mvk.workspace_size(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                   maxlen, p)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    eager = [torch.empty_like(l.q) for l in wl.layers]
    run_step(wl, bt, cl, slots, eager, p, ws, maxlen, fused)
    torch.cuda.synchronize()

    graphed = [torch.empty_like(l.q) for l in wl.layers]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_step(wl, bt, cl, slots, graphed, p, ws, maxlen, fused)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_step(wl, bt, cl, slots, graphed, p, ws, maxlen, fused)
    for rep in range(3):
        for o in graphed:
            o.fill_(float("nan"))
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()           # unrelated eager work, then a sync
        g.replay()
        torch.cuda.synchronize()
        for li, (a, b) in enumerate(zip(eager, graphed)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (case, rep)
            err = max_err(b, refs[li], wl.dtype)
            assert err <= TOL[wl.dtype], (case, rep, li, err)
        for l, (kc, vc) in zip(wl.layers, pools):   # the replayed writes land as the oracle's
            assert np.array_equal(bits(l.k_cache), kc) and np.array_equal(bits(l.v_cache), vc)
    print(f"graph {case} fused={fused}: 3 replays x {len(refs)} layers match eager bitwise and "
          f"the oracle (last max abs err {err:.3e})", flush=True)


def replay_and_check(capture, prepare, pairs, label, check=None):
    """Warm up on a side stream, capture, then replay three times, each after
    prepare() (clobbering the outputs), unrelated eager work and a sync,
    comparing every (eager, graphed) pair bit for bit and calling check()
    (the oracle comparison) after every replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        capture()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capture()
    for rep in range(3):
        prepare()
        x = torch.randn(512, 512, device="cuda")
        (x @ x).sum().item()
        g.replay()
        torch.cuda.synchronize()
        for a, b in pairs:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (label, rep)
        if check is not None:
            check(rep)


@pytest.mark.parametrize("partition_tokens", [0, 64], ids=["single_pass", "split_merge"])
def test_multi_query_graph_replay_matches_eager(partition_tokens):
    lens = [300, 41, 7, 1000, 96]
    wl = W.make_custom("g", "bf16", lens, 16, 4, 128, sum(-(-L // 16) for L in lens) + 4, 31)
    q, qs = W.make_queries(wl, [5, 3, 7, 2, 6], seed=32)
    maxlen, maxq = wl.max_context_len, 7
    lc = wl.layers[0]
    ref = oracle.paged_multi_query(bits(q), bits(lc.k_cache), bits(lc.v_cache),
                                   wl.block_tables.numpy(), wl.context_lens.numpy(), qs.numpy(),
                                   wl.scale, wl.dtype)
    wl, q, qs = wl.to("cuda"), q.to("cuda"), qs.to("cuda")
    layer = wl.layers[0]
    nbytes, _ = mvk.multi_query_workspace_size(wl.num_seqs, q.shape[0], maxq, wl.num_q_heads,
                                               wl.num_kv_heads, wl.head_dim, maxlen,
                                               partition_tokens)
    ws = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device="cuda")

    def call(out):
        mvk.paged_attention_multi_query(q, layer.k_cache, layer.v_cache, wl.block_tables,
                                        wl.context_lens, qs, wl.scale, max_query_len=maxq,
                                        max_context_len=maxlen, out=out,
                                        partition_tokens=partition_tokens, workspace=ws)
    eager = torch.empty_like(q)
    call(eager)
    torch.cuda.synchronize()
    graphed = torch.empty_like(q)
    def check(rep):
        err = max_err(graphed, ref, "bf16")
        assert err <= TOL["bf16"], (partition_tokens, rep, err)
    replay_and_check(lambda: call(graphed), lambda: graphed.fill_(float("nan")),
                     [(eager, graphed)], f"mq p={partition_tokens}", check)


def test_planned_multi_query_graph_replay_matches_eager():
    """The step the benchmark captures for a planned multi-query batch: the
    plan, then the planned call, replayed; every replay against eager and the
    oracle."""
    lens = [300, 41, 7, 1000, 96]
    wl = W.make_custom("g", "bf16", lens, 16, 8, 128, sum(-(-L // 16) for L in lens) + 4, 34)
    q, qs = W.make_queries(wl, [5, 3, 7, 2, 6], seed=35)
    maxlen, maxq = wl.max_context_len, 7
    lc = wl.layers[0]
    ref = oracle.paged_multi_query(bits(q), bits(lc.k_cache), bits(lc.v_cache),
                                   wl.block_tables.numpy(), wl.context_lens.numpy(), qs.numpy(),
                                   wl.scale, wl.dtype)
    wl, q, qs = wl.to("cuda"), q.to("cuda"), qs.to("cuda")
    layer = wl.layers[0]
    plan = mvk.make_plan(wl.block_tables, wl.context_lens, wl.num_q_heads, wl.num_kv_heads,
                         wl.head_dim, maxlen)

    def call(out):
        mvk.make_plan(wl.block_tables, wl.context_lens, wl.num_q_heads, wl.num_kv_heads,
                      wl.head_dim, maxlen, plan=plan)
        mvk.paged_attention_multi_query_planned(q, layer.k_cache, layer.v_cache, plan, qs,
                                                wl.num_seqs, wl.scale, maxq, maxlen, out=out)
    eager = torch.empty_like(q)
    call(eager)
    torch.cuda.synchronize()
    assert max_err(eager, ref, "bf16") <= TOL["bf16"]
    graphed = torch.empty_like(q)

    def check(rep):
        err = max_err(graphed, ref, "bf16")
        assert err <= TOL["bf16"], (rep, err)
    replay_and_check(lambda: call(graphed), lambda: graphed.fill_(float("nan")),
                     [(eager, graphed)], "planned mq", check)


def test_prefill_graph_replay_matches_eager():
    pf = W.make_prefill("f16", [200, 17, 64, 129], 16, 2, 64, seed=33)
    maxlen = pf.max_seqlen
    ref = oracle.prefill_attention(bits(pf.q), bits(pf.key), bits(pf.value), pf.cu_seqlens.numpy(),
                                   pf.scale, "f16")
    kc_ref, vc_ref = oracle.cache_write(bits(pf.k_cache), bits(pf.v_cache), bits(pf.key),
                                        bits(pf.value), pf.slot_mapping.numpy())
    g = pf.to("cuda")
    k0, v0 = g.k_cache.clone(), g.v_cache.clone()

    def call(out):
        mvk.prefill_attention(g.q, g.key, g.value, g.cu_seqlens, g.scale, max_seqlen=maxlen,
                              k_cache=g.k_cache, v_cache=g.v_cache, slot_mapping=g.slot_mapping,
                              out=out)
    eager = torch.empty_like(g.q)
    call(eager)
    torch.cuda.synchronize()
    k_eager, v_eager = g.k_cache.clone(), g.v_cache.clone()
    assert not torch.equal(k_eager.view(torch.int16), k0.view(torch.int16))
    graphed = torch.empty_like(g.q)

    def prepare():   # the pools as before the call, the output clobbered
        g.k_cache.copy_(k0)
        g.v_cache.copy_(v0)
        graphed.fill_(float("nan"))
    def check(rep):
        err = max_err(graphed, ref, "f16")
        assert err <= TOL["f16"], (rep, err)
        assert np.array_equal(bits(g.k_cache), kc_ref) and np.array_equal(bits(g.v_cache), vc_ref)
    prepare()
    replay_and_check(lambda: call(graphed), prepare,
                     [(eager, graphed), (k_eager, g.k_cache), (v_eager, g.v_cache)], "prefill",
                     check)

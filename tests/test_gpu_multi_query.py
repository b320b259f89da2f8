"""Multi-query paged attention (several new tokens per sequence, causal among
them) on the GPU vs the fp64 CPU oracle, through the C ABI.

Tolerance as for decode: max |gpu - oracle| <= 2e-3 (fp16) / 1.5e-2 (bf16)
over every output row. Bit-for-bit: one new token per sequence equals the
decode call on the MFMA shapes, relabelling physical blocks, repeated calls,
NaN in never-read slots."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_206_amd as mvk
import workloads as W
from gpu_helpers import TOL, bits, max_err

pytestmark = pytest.mark.gpu


def mq_case(dtype, lens, news, hq, hkv, d, seed, extra=4):
    nb = sum(-(-L // 16) for L in lens) + extra
    wl = W.make_custom("mq", dtype, lens, hq, hkv, d, max(nb, 1), seed)
    q, qs = W.make_queries(wl, news, seed + 1)
    return wl, q, qs


def oracle_mq(wl, q, qs, seqs=None):
    layer = wl.layers[0]
    bt, cl, qs_np = wl.block_tables.numpy(), wl.context_lens.numpy(), qs.numpy()
    qb = bits(q)
    if seqs is not None:   # a subset of sequences, with their own row ranges
        rows = np.concatenate([np.arange(qs_np[s], qs_np[s + 1]) for s in seqs]).astype(np.int64)
        news = np.array([qs_np[s + 1] - qs_np[s] for s in seqs])
        sub_qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
        ref = oracle.paged_multi_query(qb[rows], bits(layer.k_cache), bits(layer.v_cache),
                                       bt[seqs], cl[seqs], sub_qs, wl.scale, wl.dtype)
        return ref, rows
    ref = oracle.paged_multi_query(qb, bits(layer.k_cache), bits(layer.v_cache), bt, cl, qs_np,
                                   wl.scale, wl.dtype)
    return ref, None


def gpu_mq(wl_gpu, q, qs, partition_tokens=0, out=None):
    layer = wl_gpu.layers[0]
    return mvk.paged_attention_multi_query(q, layer.k_cache, layer.v_cache, wl_gpu.block_tables,
                                           wl_gpu.context_lens, qs, wl_gpu.scale,
                                           max_context_len=wl_gpu.max_context_len,
                                           partition_tokens=partition_tokens, out=out)


def parity(wl, q, qs, partition_tokens=0, seqs=None):
    out = gpu_mq(wl.to("cuda"), q.to("cuda"), qs.to("cuda"), partition_tokens)
    torch.cuda.synchronize()
    ref, rows = oracle_mq(wl, q, qs, seqs)
    got = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    err = max_err(got, ref, wl.dtype)
    assert err <= TOL[wl.dtype], f"max abs err {err:.3e} > {TOL[wl.dtype]}"
    return out, err


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_sweep_dtype_headdim_group(dtype, d, g):
    # new-token counts 1..9 (several row groups of 16 for g >= 2), none, and a
    # sequence that is entirely new (pure prefill of 17 tokens)
    lens = [1, 15, 16, 17, 100, 333, 64, 9, 40, 17]
    news = [1, 3, 16, 5, 9, 4, 0, 9, 2, 17]
    wl, q, qs = mq_case(dtype, lens, news, 2 * g, 2, d, seed=g * 10 + d)
    print(f"{dtype} d={d} g={g}", flush=True)
    parity(wl, q, qs)
    parity(wl, q, qs, partition_tokens=32)   # split path: partitions + merge


@pytest.mark.parametrize("p", [16, 48, 128, 512])
def test_partition_boundaries_inside_the_new_tokens(p):
    """Contexts whose new tokens straddle partition boundaries: some rows see
    nothing of the last partition and must weigh nothing there."""
    lens = [p + 2, 2 * p + 1, 3 * p, p, 700, 1025]
    news = [4, 3, 2, 5, 8, 1]
    wl, q, qs = mq_case("bf16", lens, news, 8, 2, 128, seed=p)
    single, _ = parity(wl, q, qs, partition_tokens=2048)
    split, _ = parity(wl, q, qs, partition_tokens=p)
    diff = np.abs(oracle.widen(bits(single), "bf16") - oracle.widen(bits(split), "bf16")).max()
    assert diff <= TOL["bf16"]


@pytest.mark.parametrize("dtype,d,g", [("f16", 64, 8), ("bf16", 128, 4), ("bf16", 128, 2)])
def test_one_new_token_equals_decode_bitwise(dtype, d, g):
    """With n = 1 everywhere the rows are the decode call's rows; on the MFMA
    shapes (g >= 2) the arithmetic is the same, so the bits are too."""
    lens = [1, 30, 64, 17, 250, 2]
    wl, q, qs = mq_case(dtype, lens, [1] * len(lens), 2 * g, 2, d, seed=50 + g)
    wl.layers[0].q = q
    gw = wl.to("cuda")
    a = gpu_mq(gw, gw.layers[0].q, qs.to("cuda"))
    b = mvk.paged_attention_decode(gw.layers[0].q, gw.layers[0].k_cache, gw.layers[0].v_cache,
                                   gw.block_tables, gw.context_lens, gw.scale,
                                   max_context_len=gw.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_permutation_invariance_and_determinism_bitwise():
    wl, q, qs = mq_case("bf16", [40, 7, 250, 33], [5, 7, 2, 8], 8, 4, 64, seed=6, extra=20)
    gw, qg, qsg = wl.to("cuda"), q.to("cuda"), qs.to("cuda")
    a = gpu_mq(gw, qg, qsg)
    a2 = gpu_mq(gw, qg, qsg)
    pi = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(61))
    layer = wl.layers[0]
    k2, v2 = torch.empty_like(layer.k_cache), torch.empty_like(layer.v_cache)
    k2[pi], v2[pi] = layer.k_cache, layer.v_cache
    bt = wl.block_tables.clone()
    used = bt >= 0
    bt[used] = pi[bt[used].long()].to(torch.int32)
    wl2 = W.Workload("p", wl.dtype, wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                     wl.num_blocks, wl.scale, wl.context_lens, bt, [W.Layer(layer.q, k2, v2)])
    b = gpu_mq(wl2.to("cuda"), qg, qsg)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), a2.view(torch.int16))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_nan_in_unread_slots_does_not_leak():
    for dtype, d, g in (("f16", 64, 8), ("bf16", 128, 2)):
        wl, q, qs = mq_case(dtype, [1, 5, 16, 17, 31, 200], [1, 5, 3, 17, 2, 6], 2 * g, 2, d,
                            seed=8, extra=6)
        clean, _ = parity(wl, q, qs)
        W.poison_unread(wl)
        poisoned, _ = parity(wl, q, qs)
        assert torch.equal(clean.view(torch.int16), poisoned.view(torch.int16))
        parity(wl, q, qs, partition_tokens=32)


def test_large_logits():
    wl, q, qs = mq_case("f16", [500, 37, 9, 2000], [6, 3, 9, 4], 8, 2, 128, seed=10)
    q.mul_(20.0)
    parity(wl, q, qs)
    parity(wl, q, qs, partition_tokens=64)


def test_output_rows_outside_the_queries_untouched():
    """out may be a slice of a bigger buffer; only the T query rows are written."""
    wl, q, qs = mq_case("bf16", [40, 80], [3, 2], 4, 2, 64, seed=12)
    big = torch.zeros((7, 4, 64), dtype=torch.bfloat16, device="cuda")
    out = big[1:6]
    gpu_mq(wl.to("cuda"), q.to("cuda"), qs.to("cuda"), out=out)
    torch.cuda.synchronize()
    assert torch.all(big[0] == 0) and torch.all(big[6] == 0)
    ref, _ = oracle_mq(wl, q, qs)
    assert max_err(out, ref, "bf16") <= TOL["bf16"]


def test_speculative_verification_qwen3_shape():
    """The Qwen3-0.6B decode shape with 4 draft tokens per sequence (5 new
    tokens: the last accepted one and the drafts), full size, every sequence
    checked against the oracle."""
    wl = W.make("qwen3", layers=1)
    q, qs = W.make_queries(wl, [5] * wl.num_seqs, seed=77)
    parity(wl, q, qs)


def test_speculative_verification_tinyllama_shape_sampled():
    """The TinyLlama-1.1B decode shape (256 x 512-2048 tokens, g = 8) with 2
    draft tokens (3 new tokens per sequence), full size and in the launch
    configuration the benchmark times (single pass, dispatched longest
    first); 32 sequences checked against the oracle."""
    wl = W.make("tinyllama")
    q, qs = W.make_queries(wl, [3] * wl.num_seqs, seed=78)
    parity(wl, q, qs, seqs=list(range(0, 256, 8)))


def test_speculative_verification_llama7b_long_sampled():
    """The Llama-7B long-context shape (32 x 32768 tokens, 16 sequences sharing
    a 16384-token prefix) with 4 draft tokens, full size, in the benchmark's
    launch configuration (split, shared prefix blocks kept cached); two
    prefix sharers and two private sequences checked."""
    wl = W.make("llama7b_long")
    q, qs = W.make_queries(wl, [5] * wl.num_seqs, seed=79)
    parity(wl, q, qs, seqs=[0, 15, 16, 31])


def test_long_context_verification_sampled():
    """Long contexts (8 x 16384 tokens, 5 new each) through the split path;
    4 sequences are checked against the oracle."""
    lens = [16384] * 8
    wl, q, qs = mq_case("bf16", lens, [5] * 8, 32, 8, 128, seed=90)
    parity(wl, q, qs, seqs=[0, 3, 5, 7])


@pytest.mark.parametrize("g,d,dtype", [(4, 128, "bf16"), (8, 64, "f16")])
def test_maximum_query_length(g, d, dtype):
    """1024 new tokens per sequence, the most one call accepts: one sequence
    entirely new (1024 tokens), one with a 476-token cached prefix, next to a
    one-token decode row; many row groups per (sequence, KV head); single pass
    and split."""
    wl, q, qs = mq_case(dtype, [1500, 1024, 40], [1024, 1024, 1], 2 * g, 2, d, seed=71)
    parity(wl, q, qs)
    parity(wl, q, qs, partition_tokens=256)
    with pytest.raises(mvk.MvkError):   # one more token than a call accepts
        mvk.multi_query_workspace_size(3, q.shape[0], 1025, 2 * g, 2, d, 1500)


@pytest.mark.parametrize("num_seqs", [1, 65, 256, 257])
@pytest.mark.parametrize("dtype,d,g", [("f16", 64, 8), ("bf16", 128, 2)])
def test_longest_first_order_writes_every_row(num_seqs, dtype, d, g):
    """Single-pass multi-query grids of up to 256 sequences with one row group
    and a longest context of at least 1024 tokens are dispatched longest
    sequence first (each workgroup ranks the batch); every row must be written
    once with the right value whatever the ties and empty contexts (257
    sequences keep batch order). `out` starts as NaN, so an unwritten row fails."""
    rng = np.random.default_rng(num_seqs * 7 + g)
    lens = [int(x) for x in rng.choice([0, 3, 16, 17, 100, 100, 250, 1100], size=num_seqs)]
    lens[0] = 1100
    news = [min(L, int(rng.integers(0, 3))) for L in lens]
    news[0] = 2
    wl, q, qs = mq_case(dtype, lens, news, 2 * g, 2, d, seed=num_seqs + g)
    print(f"mq longest-first S={num_seqs} {dtype} d={d} g={g}", flush=True)
    wl_gpu = wl.to("cuda")
    out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
    gpu_mq(wl_gpu, q.to("cuda"), qs.to("cuda"), partition_tokens=4096, out=out)
    torch.cuda.synchronize()
    ref, _ = oracle_mq(wl, q, qs)
    err = max_err(out, ref, wl.dtype)
    assert err <= TOL[wl.dtype], f"max abs err {err:.3e} > {TOL[wl.dtype]}"


def test_shared_prefix_equals_copied_blocks_bitwise():
    """Sequences whose tables share their first blocks (a common prompt): the
    split kernels keep blocks shared with a neighbouring sequence cached
    instead of streaming them, which must change nothing in the result - the
    same call over private copies of those blocks gives the same bits."""
    lens, news = [600, 700, 517, 33], [3, 1, 4, 2]
    shared = W.make_custom("s", "bf16", lens, 8, 2, 128, 200, seed=9,
                           shared_prefix=({0, 1, 2, 3}, 2))
    q, qs = W.make_queries(shared, news, 10)
    layer = shared.layers[0]
    bt = shared.block_tables.clone()
    k, v = layer.k_cache.clone(), layer.v_cache.clone()
    used = set(int(x) for x in shared.used_block_ids())
    free = [b for b in range(shared.num_blocks) if b not in used]
    for s in range(1, 4):
        for b in range(2):
            src = int(bt[s, b])
            dst = free.pop()
            k[dst], v[dst] = k[src], v[src]
            bt[s, b] = dst
    copied = W.Workload("c", "bf16", 4, 8, 2, 128, shared.num_blocks, shared.scale,
                        shared.context_lens, bt, [W.Layer(layer.q, k, v)])
    for p in (0, 128):
        a = gpu_mq(shared.to("cuda"), q.to("cuda"), qs.to("cuda"), partition_tokens=p)
        b = gpu_mq(copied.to("cuda"), q.to("cuda"), qs.to("cuda"), partition_tokens=p)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    parity(shared, q, qs, partition_tokens=128)

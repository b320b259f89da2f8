"""Prefill attention (causal self-attention of new prompts, with the fused
cache write) on the GPU vs the fp64 CPU oracle, through the C ABI.

Attention: max |gpu - oracle| <= 2e-3 (fp16) / 1.5e-2 (bf16) over every
output row. Cache write: whole pools bit-exact against the oracle's write.
Bit-for-bit: repeated calls, and the output with and without the write."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_206_amd as mvk
import workloads as W
from gpu_helpers import TOL, bits, max_err

pytestmark = pytest.mark.gpu


def oracle_prefill(pf, rows=None):
    ref = oracle.prefill_attention(bits(pf.q), bits(pf.key), bits(pf.value), pf.cu_seqlens.numpy(),
                                   pf.scale, pf.dtype)
    return ref if rows is None else ref[rows]


def gpu_prefill(g, write=True, out=None):
    kw = dict(k_cache=g.k_cache, v_cache=g.v_cache, slot_mapping=g.slot_mapping) if write else {}
    return mvk.prefill_attention(g.q, g.key, g.value, g.cu_seqlens, g.scale,
                                 max_seqlen=g.max_seqlen, out=out, **kw)


def check(pf, write=True):
    g = pf.to("cuda")
    out = gpu_prefill(g, write)
    torch.cuda.synchronize()
    err = max_err(out, oracle_prefill(pf), pf.dtype)
    assert err <= TOL[pf.dtype], f"max abs err {err:.3e} > {TOL[pf.dtype]}"
    return g, out


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_sweep_dtype_headdim_group(dtype, d, g):
    # lengths around the 16-token block, the 64-token query tile and K/V tile
    lens = [1, 15, 16, 17, 63, 64, 65, 130, 3]
    pf = W.make_prefill(dtype, lens, 2 * g, 2, d, seed=g * 10 + d)
    print(f"{dtype} d={d} g={g}", flush=True)
    check(pf)


@pytest.mark.parametrize("dtype,hq", [("bf16", 8), ("f16", 2)])
def test_long_batch_with_ragged_prompts(dtype, hq):
    """head_dim 128, one prompt of 2100 tokens among short ones around the
    64-token tiles and 128-token query ranges, with empty and one-token
    prompts: every row against the oracle and the pools bit-exact."""
    lens = [2100, 0, 1, 255, 256, 257, 511, 300]
    pf = W.make_prefill(dtype, lens, hq, 2, 128, seed=12 + hq)
    before_k, before_v = bits(pf.k_cache), bits(pf.v_cache)
    g, _ = check(pf)
    k_ref, v_ref = oracle.cache_write(before_k, before_v, bits(pf.key), bits(pf.value),
                                      pf.slot_mapping.numpy())
    assert np.array_equal(bits(g.k_cache), k_ref)
    assert np.array_equal(bits(g.v_cache), v_ref)


def test_cache_write_is_bit_exact():
    """The pools after the call equal the oracle's write of every row into its
    slot (a negative slot is skipped), everything else untouched."""
    pf = W.make_prefill("bf16", [37, 5, 70], 8, 2, 128, seed=3, extra_blocks=6)
    pf.slot_mapping[4] = -1
    before_k, before_v = bits(pf.k_cache), bits(pf.v_cache)
    g, _ = check(pf)
    k_ref, v_ref = oracle.cache_write(before_k, before_v, bits(pf.key), bits(pf.value),
                                      pf.slot_mapping.numpy())
    assert np.array_equal(bits(g.k_cache), k_ref)
    assert np.array_equal(bits(g.v_cache), v_ref)


def test_write_does_not_change_attention_and_is_deterministic():
    pf = W.make_prefill("f16", [100, 33, 7], 16, 4, 64, seed=4)
    g = pf.to("cuda")
    a = gpu_prefill(g, write=False)
    b = gpu_prefill(g, write=True)
    c = gpu_prefill(g, write=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(b.view(torch.int16), c.view(torch.int16))


def test_equals_multi_query_with_every_token_new():
    """After the write, the pools hold the prompts, and the multi-query call with
    n = L over them computes the same attention."""
    lens = [40, 97, 16]
    pf = W.make_prefill("bf16", lens, 8, 2, 128, seed=5)
    g, out = check(pf)
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    mq = mvk.paged_attention_multi_query(g.q, g.k_cache, g.v_cache, g.block_tables, cl,
                                         g.cu_seqlens, g.scale, max_query_len=max(lens),
                                         max_context_len=max(lens))
    torch.cuda.synchronize()
    diff = np.abs(oracle.widen(bits(out), "bf16") - oracle.widen(bits(mq), "bf16")).max()
    assert diff <= TOL["bf16"]


def test_large_logits_and_output_slice():
    pf = W.make_prefill("f16", [90, 12], 8, 2, 64, seed=6)
    pf.q.mul_(20.0)
    g = pf.to("cuda")
    big = torch.zeros((pf.q.shape[0] + 2, 8, 64), dtype=torch.float16, device="cuda")
    out = big[1:-1]
    gpu_prefill(g, out=out)
    torch.cuda.synchronize()
    assert torch.all(big[0] == 0) and torch.all(big[-1] == 0)
    assert max_err(out, oracle_prefill(pf), "f16") <= TOL["f16"]


def test_long_prompt_sampled_rows():
    """A 2048-token prompt (TinyLlama shape): rows from every 64-token tile,
    first and last included. Each sampled row r is the oracle's multi-query
    row with one new token at position r, over the oracle's own cache write of
    the prompt."""
    pf = W.make_prefill("f16", [2048], 32, 4, 64, seed=7)
    g = pf.to("cuda")
    out = gpu_prefill(g)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 2048, 61), [0, 63, 64, 2047]]))
    q = bits(pf.q)
    kc, vc = oracle.cache_write(bits(pf.k_cache), bits(pf.v_cache), bits(pf.key), bits(pf.value),
                                pf.slot_mapping.numpy())
    bt = pf.block_tables.numpy()
    ref = np.stack([oracle.paged_multi_query(q[r:r + 1], kc, vc, bt,
                                             np.array([r + 1], dtype=np.int32),
                                             np.array([0, 1], dtype=np.int32), pf.scale, "f16")[0]
                    for r in rows])
    err = max_err(out[torch.as_tensor(rows, device="cuda")], ref, "f16")
    assert err <= TOL["f16"]


def test_empty_prompts_and_a_loose_length_bound():
    """Zero-length prompts between others write nothing and produce no rows;
    a max_seqlen above every prompt length only adds workgroups that exit."""
    pf = W.make_prefill("bf16", [0, 37, 0, 130, 5, 0], 8, 2, 64, seed=8)
    before_k, before_v = bits(pf.k_cache), bits(pf.v_cache)
    g = pf.to("cuda")
    out = mvk.prefill_attention(g.q, g.key, g.value, g.cu_seqlens, g.scale, max_seqlen=600,
                                k_cache=g.k_cache, v_cache=g.v_cache, slot_mapping=g.slot_mapping)
    torch.cuda.synchronize()
    assert max_err(out, oracle_prefill(pf), "bf16") <= TOL["bf16"]
    k_ref, v_ref = oracle.cache_write(before_k, before_v, bits(pf.key), bits(pf.value),
                                      pf.slot_mapping.numpy())
    assert np.array_equal(bits(g.k_cache), k_ref)
    assert np.array_equal(bits(g.v_cache), v_ref)


def test_long_prompt_llama_shape_sampled_rows():
    """An 8192-token prompt in the Llama-7B shape (32 q / 8 kv heads, head_dim
    128, bf16): rows on both sides of every kind of boundary (16-row tiles,
    64-token K/V tiles, 128-token workgroup ranges) and spread over the
    prompt, each checked against a single-row oracle call over the oracle's
    own cache write of the prompt."""
    pf = W.make_prefill("bf16", [8192], 32, 8, 128, seed=9)
    g = pf.to("cuda")
    out = gpu_prefill(g)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 8192, 509), [0, 15, 16, 63, 64, 127, 128, 4095,
                                                               4096, 8063, 8064, 8191]]))
    q = bits(pf.q)
    kc, vc = oracle.cache_write(bits(pf.k_cache), bits(pf.v_cache), bits(pf.key), bits(pf.value),
                                pf.slot_mapping.numpy())
    bt = pf.block_tables.numpy()
    ref = np.stack([oracle.paged_multi_query(q[r:r + 1], kc, vc, bt,
                                             np.array([r + 1], dtype=np.int32),
                                             np.array([0, 1], dtype=np.int32), pf.scale, "bf16")[0]
                    for r in rows])
    err = max_err(out[torch.as_tensor(rows, device="cuda")], ref, "bf16")
    assert err <= TOL["bf16"]


def test_llama_shape_full_batch_sampled_rows():
    """The benchmark's Llama-7B prefill call at full size (32 prompts x 4096
    tokens, 32 q / 8 kv heads, head_dim 128, bf16, fused cache write, the
    library's launch configuration): rows at tile and range boundaries of the
    first, a middle and the last prompt, each against a single-row oracle call
    over the oracle's own cache write; the whole pools bit-exact."""
    S, n = 32, 4096
    pf = W.make_prefill("bf16", [n] * S, 32, 8, 128, seed=11)
    g = pf.to("cuda")
    out = gpu_prefill(g)
    torch.cuda.synchronize()
    q = bits(pf.q)
    kc, vc = oracle.cache_write(bits(pf.k_cache), bits(pf.v_cache), bits(pf.key), bits(pf.value),
                                pf.slot_mapping.numpy())
    assert np.array_equal(bits(g.k_cache), kc) and np.array_equal(bits(g.v_cache), vc)
    bt = pf.block_tables.numpy()
    cu = pf.cu_seqlens.numpy()
    picks = [(p, r) for p in (0, 17, S - 1) for r in (0, 15, 16, 127, 128, 2047, 2048, 4095)]
    ref = np.stack([oracle.paged_multi_query(q[cu[p] + r:cu[p] + r + 1], kc, vc, bt[p:p + 1],
                                             np.array([r + 1], dtype=np.int32),
                                             np.array([0, 1], dtype=np.int32), pf.scale, "bf16")[0]
                    for p, r in picks])
    rows = torch.as_tensor([int(cu[p]) + r for p, r in picks], device="cuda")
    err = max_err(out[rows], ref, "bf16")
    assert err <= TOL["bf16"], f"max abs err {err:.3e}"

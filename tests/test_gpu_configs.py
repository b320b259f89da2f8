"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (library-chosen partitioning, the step's cache write fused into the
decode call) and with the write as its own call, checked against the fp64
oracle on sampled sequences. Each step is the cache write of the step's new
token rows followed by decode, on both sides."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_206_amd as mvk
import workloads as W
from gpu_helpers import TOL, bits, max_err

pytestmark = pytest.mark.gpu


def step_and_check(wl, layer_idx, seqs, fused=False):
    layer = wl.layers[layer_idx]
    kc_host, vc_host = bits(layer.k_cache), bits(layer.v_cache)
    q_host = bits(layer.q)
    bt = wl.block_tables.numpy()
    cl = wl.context_lens.numpy()
    if layer.key is not None:
        kc_host, vc_host = oracle.cache_write(kc_host, vc_host, bits(layer.key), bits(layer.value),
                                              wl.slot_mapping.numpy())
    ref = oracle.paged_decode(q_host[seqs], kc_host, vc_host, bt[seqs], cl[seqs], wl.scale,
                              wl.dtype)
    gl = W.Layer(*(None if t is None else t.cuda() for t in
                   (layer.q, layer.k_cache, layer.v_cache, layer.key, layer.value)))
    bt_g, cl_g = wl.block_tables.cuda(), wl.context_lens.cuda()
    if gl.key is not None and fused:    # the benchmark's call: write fused into decode
        out = mvk.paged_attention_decode(gl.q, gl.k_cache, gl.v_cache, bt_g, cl_g, wl.scale,
                                         max_context_len=wl.max_context_len, new_key=gl.key,
                                         new_value=gl.value, slot_mapping=wl.slot_mapping.cuda())
    else:
        if gl.key is not None:
            mvk.reshape_and_cache(gl.key, gl.value, gl.k_cache, gl.v_cache,
                                  wl.slot_mapping.cuda())
        out = mvk.paged_attention_decode(gl.q, gl.k_cache, gl.v_cache, bt_g, cl_g, wl.scale,
                                         max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    if gl.key is not None:   # the write itself is bit-exact over the whole pool
        assert np.array_equal(bits(gl.k_cache), kc_host)
        assert np.array_equal(bits(gl.v_cache), vc_host)
    err = max_err(out, ref, wl.dtype, seqs)
    print(f"{wl.name} layer {layer_idx} fused={fused}: {len(seqs)} seqs checked, "
          f"max abs err {err:.3e}, "
          f"max |out| {np.abs(ref).max():.3f}", flush=True)
    assert err <= TOL[wl.dtype]


FUSED = pytest.mark.parametrize("fused", [True, False], ids=["fused_write", "separate_write"])


@FUSED
def test_qwen3_shaped_all_sequences(fused):
    wl = W.make("qwen3", layers=2)
    for layer_idx in range(2):
        step_and_check(wl, layer_idx, np.arange(wl.num_seqs), fused)


@FUSED
def test_tinyllama_shaped_sampled(fused):
    wl = W.make("tinyllama")
    step_and_check(wl, 0, np.arange(0, 256, 8), fused)


@FUSED
def test_llama7b_long_context_sampled(fused):
    wl = W.make("llama7b_long")
    step_and_check(wl, 0, np.array([0, 15, 16, 31]), fused)   # two prefix sharers, two private


@FUSED
def test_skewed_batch_sampled(fused):
    wl = W.make("skewed")
    lens = wl.context_lens
    longest = int(torch.argmax(lens))
    singles = torch.nonzero(lens == 1).flatten()[:3].tolist()
    g = torch.Generator().manual_seed(44)
    others = torch.randperm(wl.num_seqs, generator=g)[:8].tolist()
    seqs = np.array(sorted(set([longest] + singles + others)))
    step_and_check(wl, 0, seqs, fused)

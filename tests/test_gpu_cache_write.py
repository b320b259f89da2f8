"""Cache write on the GPU: whole-pool bit equality with the oracle, guard bands
around the pools untouched (no stray writes), through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_206_amd as mvk
import workloads as W
from gpu_helpers import bits

pytestmark = pytest.mark.gpu

GUARD = 2  # guard blocks before and after each pool


def guarded_pool(host_pool: torch.Tensor, pattern: int):
    nb = host_pool.shape[0]
    big = torch.empty((nb + 2 * GUARD, *host_pool.shape[1:]), dtype=host_pool.dtype)
    big.view(torch.int16).fill_(pattern)
    big[GUARD:GUARD + nb] = host_pool
    big = big.cuda()
    return big, big[GUARD:GUARD + nb]


def check_write(k_host, v_host, key, value, slots):
    dt = "f16" if k_host.dtype == torch.float16 else "bf16"
    kbig, kview = guarded_pool(k_host, 0x1234)
    vbig, vview = guarded_pool(v_host, 0x4321)
    mvk.reshape_and_cache(key.cuda(), value.cuda(), kview, vview, slots.cuda())
    torch.cuda.synchronize()
    ek, ev = oracle.cache_write(bits(k_host), bits(v_host), bits(key), bits(value), slots.numpy())
    gk, gv = bits(kbig), bits(vbig)
    nb = k_host.shape[0]
    assert np.array_equal(gk[GUARD:GUARD + nb], ek), f"K pool differs ({dt})"
    assert np.array_equal(gv[GUARD:GUARD + nb], ev), f"V pool differs ({dt})"
    assert np.all(gk[:GUARD] == 0x1234) and np.all(gk[GUARD + nb:] == 0x1234), "K guard written"
    assert np.all(gv[:GUARD] == 0x4321) and np.all(gv[GUARD + nb:] == 0x4321), "V guard written"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hkv,d", [(1, 64), (2, 64), (4, 128), (8, 128), (3, 64)])
def test_cache_write_random_slots(dtype, hkv, d):
    g = torch.Generator().manual_seed(hkv * 1000 + d)
    nb, T = 40, 300
    k = W.randn_storage((nb, 16, hkv, d), dtype, g)
    v = W.randn_storage((nb, 16, hkv, d), dtype, g)
    key = W.randn_storage((T, hkv, d), dtype, g)
    value = W.randn_storage((T, hkv, d), dtype, g)
    slots = torch.randperm(nb * 16, generator=g)[:T].to(torch.int32)
    slots[::7] = -1                      # padding
    slots[5] = nb * 16                   # one past the pool: must be skipped
    slots[6] = nb * 16 + 100
    expect_slots = slots.clone()
    expect_slots[5] = -1
    expect_slots[6] = -1
    kbig, kview = guarded_pool(k, 0x1234)
    vbig, vview = guarded_pool(v, 0x4321)
    mvk.reshape_and_cache(key.cuda(), value.cuda(), kview, vview, slots.cuda())
    torch.cuda.synchronize()
    ek, ev = oracle.cache_write(bits(k), bits(v), bits(key), bits(value), expect_slots.numpy())
    assert np.array_equal(bits(kbig)[GUARD:GUARD + nb], ek)
    assert np.array_equal(bits(vbig)[GUARD:GUARD + nb], ev)
    assert np.all(bits(kbig)[GUARD + nb:] == 0x1234) and np.all(bits(vbig)[:GUARD] == 0x4321)


def test_cache_write_tiny_workload():
    wl = W.make("tiny")
    layer = wl.layers[0]
    check_write(layer.k_cache, layer.v_cache, layer.key, layer.value, wl.slot_mapping)


@pytest.mark.parametrize("name", ["tinyllama", "skewed", "qwen3"])
def test_cache_write_full_size(name):
    wl = W.make(name, layers=1)
    layer = wl.layers[0]
    assert layer.key.shape[0] == wl.num_seqs
    check_write(layer.k_cache, layer.v_cache, layer.key, layer.value, wl.slot_mapping)


def test_cache_write_nan_and_special_bits_copied_raw():
    """Raw copy: NaN payloads, infinities, -0 and subnormals arrive unchanged."""
    special = torch.tensor([0x7E01, 0x7C00, 0xFC00, 0x8000, 0x0001, 0x7FFF, 0xFFFF, 0x3C00],
                           dtype=torch.int32).to(torch.int16)
    key = special.repeat(4 * 64 // 8).view(4, 1, 64).view(torch.float16)
    value = torch.flip(key, dims=[2]).contiguous()
    k = torch.zeros((2, 16, 1, 64), dtype=torch.float16)
    v = torch.zeros((2, 16, 1, 64), dtype=torch.float16)
    check_write(k, v, key, value, torch.tensor([3, 31, -1, 16], dtype=torch.int32))

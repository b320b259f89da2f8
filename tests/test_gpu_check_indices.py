"""mvk_check_indices (the debug check of a step's index arrays) on the GPU,
through the C ABI: zero counts on every workload's own arrays, exact counts
for planted errors (against plain Python loops over the definition, and in
one hand-checked case against known numbers), and entries a call never reads
left uncounted."""
import numpy as np
import pytest
import torch

import paged_kv_cache_206_amd as mvk
import workloads as W

pytestmark = pytest.mark.gpu


def counted(tables, lens, maxlen, nblocks, slots=None):
    """The three counts from the definition, with plain loops."""
    tables, lens = np.asarray(tables), np.asarray(lens)
    width = tables.shape[1]
    cap = min(maxlen, 16 * width)
    bad_len = sum(1 for L in lens if L < 0 or L > maxlen)
    bad_blk = 0
    for s, L in enumerate(lens):
        n = (min(max(int(L), 0), cap) + 15) // 16
        bad_blk += sum(1 for j in range(n) if not 0 <= tables[s][j] < nblocks)
    bad_slot = 0 if slots is None else sum(1 for x in slots if x >= 16 * nblocks)
    return {"context_lens": bad_len, "block_ids": bad_blk, "slots": bad_slot}


def run(tables, lens, maxlen, nblocks, slots=None):
    t = torch.as_tensor(np.asarray(tables), dtype=torch.int32, device="cuda")
    l = torch.as_tensor(np.asarray(lens), dtype=torch.int32, device="cuda")
    sm = None if slots is None else torch.as_tensor(np.asarray(slots), dtype=torch.int32,
                                                    device="cuda")
    return mvk.check_indices(t, l, maxlen, nblocks, sm)


@pytest.mark.parametrize("name", ["tiny", "qwen3", "tinyllama", "llama7b_long", "skewed"])
def test_workload_arrays_are_clean(name):
    wl = W.make(name, values=False)
    maxlen = int(wl.context_lens.max())
    print(name, flush=True)
    got = run(wl.block_tables.numpy(), wl.context_lens.numpy(), maxlen, wl.num_blocks,
              wl.slot_mapping.numpy())
    assert got == {"context_lens": 0, "block_ids": 0, "slots": 0}


def test_hand_checked_plants():
    """Four sequences of 20, 16, 1 and 0 tokens in rows of 3 entries, a pool
    of 10 blocks: row 0 reads entries 0-1 (entry 1 = 10 is bad; entry 2 = -1
    is past its length), row 1 reads entry 0 (fine), row 2 reads entry 0
    (-4 is bad), row 3 reads nothing; one length (60) is past max_context_len
    = 48, so its row is read up to 48 tokens (3 entries: one bad, 99); slots
    159 (last of the pool) and -1 are fine, 160 is past it."""
    tables = [[3, 10, -1], [4, 77, 88], [-4, 0, 0], [5, 6, 99]]
    lens = [20, 16, 1, 60]
    got = run(tables, lens, 48, 10, [159, -1, 160, 2])
    assert got == {"context_lens": 1, "block_ids": 3, "slots": 1}


@pytest.mark.parametrize("seed", range(6))
def test_random_plants_match_the_definition(seed):
    gen = np.random.default_rng(seed)
    S = int(gen.integers(1, 700))
    width = int(gen.integers(1, 300))
    nblocks = int(gen.integers(1, 5000))
    maxlen = int(gen.integers(0, 16 * width + 40))
    lens = gen.integers(-3, maxlen + 20, S)
    tables = gen.integers(0, nblocks, (S, width))
    bad = gen.random((S, width)) < 0.01
    tables[bad] = gen.choice([-1, -100, nblocks, nblocks + 7, 2**31 - 1], bad.sum())
    slots = gen.integers(-2, 16 * nblocks + 3, int(gen.integers(0, 900)))
    print(f"seed {seed}: S={S} width={width} blocks={nblocks} maxlen={maxlen}", flush=True)
    assert run(tables, lens, maxlen, nblocks, slots) == counted(tables, lens, maxlen, nblocks, slots)


def test_empty_batch_writes_zeros():
    counts = torch.full((3,), -1, dtype=torch.int64, device="cuda")
    st = mvk.lib().mvk_check_indices(counts.data_ptr(), None, None, 0, 0, 0, None, 0, 1,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == 0
    assert counts.tolist() == [0, 0, 0]

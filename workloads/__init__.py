"""Seeded synthetic inputs for paged-attention decode and the paged cache write.

This module produces inputs only: random K/V pools, queries, new K/V rows,
block tables, context lengths and slot mappings. It holds none of the
attention arithmetic, and it is the one module that both the oracle-side code
(tests, CPU baseline) and the GPU-side code (tests, benchmark) use.

Named workloads (shapes from the model families the pages run: Qwen3-0.6B,
TinyLlama-1.1B-Chat, Llama/Mistral-7B; 16-token blocks as in the pages'
paged-cache description):

* ``tiny``      fp16, 4 seqs with lengths {1,17,32,45}, 4 q / 2 kv heads, D 64,
                32-block pool with randomly permuted physical ids, 1 layer.
* ``qwen3``     bf16, 60 seqs, lengths uniform in [64, 256], 16 q / 8 kv heads,
                D 128, 28 layers each with its own 1024-block pool, one block
                table shared by all layers, one new token per sequence per layer.
* ``tinyllama`` fp16, 256 seqs, lengths uniform in [512, 2048], 32 q / 4 kv
                heads, D 64, 32768-block pool, 256 new rows per step.
* ``llama7b_long`` bf16, 32 seqs of 32768 tokens, 32 q / 8 kv heads, D 128;
                sequences 0-15 share an identical 16384-token prefix of
                physical blocks; 65536-block pool.
* ``skewed``    bf16, 512 seqs, lengths lognormal (median 512, sigma 1) clipped
                to [1, 131072], one 131072-token sequence and 64 one-token
                sequences, 16 q / 8 kv heads, D 128, pool 98 % full, 512 new rows.

Values are N(0, 1) drawn in float32 from a seeded ``torch.Generator`` and
rounded (RNE) to the storage type. Structure (lengths, tables, slots) is
always drawn on the CPU, so it is identical on every machine; bulk values are
drawn on ``value_device`` (the CPU by default; a GPU generator for the
multi-GB pools, which is seeded but yields a different stream than the CPU).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK_SIZE = 16
TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}

SEEDS = {"tiny": 0, "qwen3": 1, "tinyllama": 2, "llama7b_long": 3, "skewed": 4}


@dataclass
class Layer:
    q: torch.Tensor        # [S, Hq, D]
    k_cache: torch.Tensor  # [NB, 16, Hkv, D]
    v_cache: torch.Tensor  # [NB, 16, Hkv, D]
    key: torch.Tensor | None = None    # [T, Hkv, D] new rows for this step
    value: torch.Tensor | None = None  # [T, Hkv, D]


@dataclass
class Workload:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    context_lens: torch.Tensor   # int32 [S]
    block_tables: torch.Tensor   # int32 [S, max_blocks], padded with -1
    layers: list = field(default_factory=list)
    slot_mapping: torch.Tensor | None = None  # int32 [T]
    block_size: int = BLOCK_SIZE

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 2

    def used_block_ids(self) -> torch.Tensor:
        """Distinct physical blocks that decode reads (for unique-byte counts)."""
        ids = []
        for s in range(self.num_seqs):
            n = -(-int(self.context_lens[s]) // self.block_size)
            ids.append(self.block_tables[s, :n])
        return torch.unique(torch.cat(ids)) if ids else torch.zeros(0, dtype=torch.int32)

    def to(self, device) -> "Workload":
        def mv(t):
            return None if t is None else t.to(device)
        layers = [Layer(mv(l.q), mv(l.k_cache), mv(l.v_cache), mv(l.key), mv(l.value))
                  for l in self.layers]
        return Workload(self.name, self.dtype, self.num_seqs, self.num_q_heads, self.num_kv_heads,
                        self.head_dim, self.num_blocks, self.scale, mv(self.context_lens),
                        mv(self.block_tables), layers, mv(self.slot_mapping), self.block_size)


# ---------------------------------------------------------------- value draws

def randn_storage(shape, dtype: str, gen: torch.Generator, device="cpu",
                  chunk: int = 1 << 26) -> torch.Tensor:
    """N(0,1) float32 draws rounded to fp16/bf16, generated in chunks so that a
    multi-GB pool never needs a float32 copy of itself."""
    out = torch.empty(shape, dtype=TORCH_DTYPE[dtype], device=device)
    flat = out.view(-1)
    for start in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - start)
        flat[start:start + n] = torch.randn(n, generator=gen, device=device,
                                            dtype=torch.float32).to(flat.dtype)
    return out


def _value_gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + 17)
    return g


# ------------------------------------------------------------ structure draws

def assign_blocks(context_lens, num_blocks: int, gen: torch.Generator, shared_prefix=None,
                  block_size: int = BLOCK_SIZE):
    """Block tables whose physical ids are taken, in order, from a seeded random
    permutation of the pool. `shared_prefix=(seqs, nblocks)` makes those
    sequences' first `nblocks` table entries identical (prefix sharing)."""
    S = len(context_lens)
    need = [-(-int(L) // block_size) for L in context_lens]
    max_blocks = max(need) if S else 1
    perm = torch.randperm(num_blocks, generator=gen).to(torch.int32)
    tables = torch.full((S, max(max_blocks, 1)), -1, dtype=torch.int32)
    cursor = 0
    prefix_ids = None
    if shared_prefix is not None:
        seqs, nshared = shared_prefix
        prefix_ids = perm[cursor:cursor + nshared]
        cursor += nshared
    for s in range(S):
        start = 0
        if prefix_ids is not None and s in shared_prefix[0]:
            k = min(len(prefix_ids), need[s])
            tables[s, :k] = prefix_ids[:k]
            start = k
        n = need[s] - start
        if cursor + n > num_blocks:
            raise ValueError("pool too small for the requested lengths")
        tables[s, start:need[s]] = perm[cursor:cursor + n]
        cursor += n
    return tables, cursor


def last_token_slots(context_lens, block_tables, block_size: int = BLOCK_SIZE) -> torch.Tensor:
    """Flat slot (physical block * block_size + offset) of each sequence's newest
    token, position L_s - 1: where that step's cache write must land so that the
    same step's decode sees it."""
    slots = []
    for s, L in enumerate(context_lens.tolist()):
        if L <= 0:
            slots.append(-1)
            continue
        t = L - 1
        slots.append(int(block_tables[s, t // block_size]) * block_size + t % block_size)
    return torch.tensor(slots, dtype=torch.int32)


def poison_unread(wl: Workload) -> None:
    """Write NaN into every pool slot that decode must never read: blocks no
    table references, and the tail of each sequence's last block."""
    bits = NAN_BITS[wl.dtype]
    used = torch.zeros(wl.num_blocks, dtype=torch.bool)
    tail = []
    for s in range(wl.num_seqs):
        L = int(wl.context_lens[s])
        n = -(-L // wl.block_size)
        used[wl.block_tables[s, :n].long()] = True
        if L % wl.block_size and n > 0:
            tail.append((int(wl.block_tables[s, n - 1]), L % wl.block_size))
    for layer in wl.layers:
        for pool in (layer.k_cache, layer.v_cache):
            raw = pool.view(torch.int16)
            idx = torch.nonzero(~used.to(pool.device)).flatten()
            raw[idx] = bits
            for blk, off in tail:
                raw[blk, off:] = bits


# -------------------------------------------------------------- named configs

def make_queries(wl: Workload, new_tokens, seed: int, device="cpu"):
    """Query rows for several new tokens per sequence: sequence s gets
    `new_tokens[s]` rows (its last new_tokens[s] context tokens). Returns
    (q [T, Hq, D] in the workload's storage type, query_start int32 [S + 1]);
    rows are N(0, 1) draws like the decode queries."""
    news = torch.as_tensor(new_tokens, dtype=torch.int64)
    if news.numel() != wl.num_seqs or bool((news < 0).any()) or \
            bool((news > wl.context_lens.to(torch.int64)).any()):
        raise ValueError("need 0 <= new_tokens[s] <= context_lens[s] for every sequence")
    query_start = torch.zeros(wl.num_seqs + 1, dtype=torch.int32)
    query_start[1:] = torch.cumsum(news, 0).to(torch.int32)
    gen = _value_gen(seed, device)
    q = randn_storage((int(query_start[-1]), wl.num_q_heads, wl.head_dim), wl.dtype, gen, device)
    return q, query_start


@dataclass
class Prefill:
    """New prompts packed along the token axis, plus a paged cache to store
    their K/V rows in: prompt s owns rows cu_seqlens[s] .. cu_seqlens[s+1]-1,
    and row r goes to flat slot slot_mapping[r] (through the prompt's own
    blocks of block_tables)."""
    dtype: str
    q: torch.Tensor            # [T, Hq, D]
    key: torch.Tensor          # [T, Hkv, D]
    value: torch.Tensor        # [T, Hkv, D]
    cu_seqlens: torch.Tensor   # int32 [S + 1]
    k_cache: torch.Tensor      # [NB, 16, Hkv, D]
    v_cache: torch.Tensor
    block_tables: torch.Tensor  # int32 [S, max_blocks]
    slot_mapping: torch.Tensor  # int32 [T]
    scale: float

    @property
    def max_seqlen(self) -> int:
        return int((self.cu_seqlens[1:] - self.cu_seqlens[:-1]).max().item()) \
            if self.cu_seqlens.numel() > 1 else 0

    def to(self, device) -> "Prefill":
        return Prefill(self.dtype, *(t.to(device) for t in (
            self.q, self.key, self.value, self.cu_seqlens, self.k_cache, self.v_cache,
            self.block_tables, self.slot_mapping)), self.scale)


def make_prefill(dtype, prompt_lens, num_q_heads, num_kv_heads, head_dim, seed,
                 extra_blocks=4, device="cpu") -> Prefill:
    """Seeded prompts: N(0, 1) q / key / value rows; each prompt gets random
    distinct physical blocks of a pool filled with N(0, 1) values, and its
    rows' slots follow its block table."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(prompt_lens, dtype=torch.int32)
    nb = int(((lens + BLOCK_SIZE - 1) // BLOCK_SIZE).sum()) + extra_blocks
    tables, _ = assign_blocks(lens, nb, gen)
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    slots = []
    for s, L in enumerate(lens.tolist()):
        for t in range(L):
            slots.append(int(tables[s, t // BLOCK_SIZE]) * BLOCK_SIZE + t % BLOCK_SIZE)
    T = int(cu[-1])
    vgen = _value_gen(seed, device)
    q = randn_storage((T, num_q_heads, head_dim), dtype, vgen, device)
    key = randn_storage((T, num_kv_heads, head_dim), dtype, vgen, device)
    value = randn_storage((T, num_kv_heads, head_dim), dtype, vgen, device)
    k_cache = randn_storage((nb, BLOCK_SIZE, num_kv_heads, head_dim), dtype, vgen, device)
    v_cache = randn_storage((nb, BLOCK_SIZE, num_kv_heads, head_dim), dtype, vgen, device)
    return Prefill(dtype, q, key, value, cu, k_cache, v_cache, tables,
                   torch.tensor(slots, dtype=torch.int32), 1.0 / math.sqrt(head_dim))


def make_custom(name, dtype, context_lens, num_q_heads, num_kv_heads, head_dim, num_blocks,
                seed, layers=1, shared_prefix=None, new_rows=True, scale=None,
                value_device="cpu", values=True) -> Workload:
    """General builder behind the named workloads and the test variants.
    `values=False` builds the structure only (no layers), for cheap checks."""
    gen = torch.Generator().manual_seed(seed)
    context_lens = torch.as_tensor(context_lens, dtype=torch.int32)
    tables, _ = assign_blocks(context_lens, num_blocks, gen, shared_prefix)
    S = len(context_lens)
    vgen = _value_gen(seed, value_device)
    wl_layers = []
    for _ in range(layers if values else 0):
        k = randn_storage((num_blocks, BLOCK_SIZE, num_kv_heads, head_dim), dtype, vgen, value_device)
        v = randn_storage((num_blocks, BLOCK_SIZE, num_kv_heads, head_dim), dtype, vgen, value_device)
        q = randn_storage((S, num_q_heads, head_dim), dtype, vgen, value_device)
        key = value = None
        if new_rows:
            key = randn_storage((S, num_kv_heads, head_dim), dtype, vgen, value_device)
            value = randn_storage((S, num_kv_heads, head_dim), dtype, vgen, value_device)
        wl_layers.append(Layer(q, k, v, key, value))
    slots = last_token_slots(context_lens, tables) if new_rows else None
    return Workload(name, dtype, S, num_q_heads, num_kv_heads, head_dim, num_blocks,
                    scale if scale is not None else 1.0 / math.sqrt(head_dim),
                    context_lens, tables, wl_layers, slots)


def _uniform_lengths(gen, n, lo, hi):
    return torch.randint(lo, hi + 1, (n,), generator=gen, dtype=torch.int64).tolist()


def make(name: str, seed: int | None = None, value_device="cpu", layers: int | None = None,
         values: bool = True) -> Workload:
    """Build a named workload. `layers` may shrink the multi-layer config for
    quick tests; the benchmark always uses the full count."""
    seed = SEEDS[name] if seed is None else seed
    lg = torch.Generator().manual_seed(seed + 7919)
    if name == "tiny":
        return make_custom(name, "f16", [1, 17, 32, 45], 4, 2, 64, 32, seed, layers=layers or 1,
                           scale=1.0 / 8.0, value_device=value_device, values=values)
    if name == "qwen3":
        lens = _uniform_lengths(lg, 60, 64, 256)
        return make_custom(name, "bf16", lens, 16, 8, 128, 1024, seed, layers=layers or 28,
                           value_device=value_device, values=values)
    if name == "tinyllama":
        lens = _uniform_lengths(lg, 256, 512, 2048)
        return make_custom(name, "f16", lens, 32, 4, 64, 32768, seed, layers=layers or 1,
                           value_device=value_device, values=values)
    if name == "llama7b_long":
        lens = [32768] * 32
        return make_custom(name, "bf16", lens, 32, 8, 128, 65536, seed, layers=layers or 1,
                           shared_prefix=(set(range(16)), 1024), value_device=value_device, values=values)
    if name == "skewed":
        lens = skewed_lengths(lg, 512)
        need = sum(-(-L // BLOCK_SIZE) for L in lens)
        nb = -(-need * 100 // 98)
        return make_custom(name, "bf16", lens, 16, 8, 128, nb, seed, layers=layers or 1,
                           value_device=value_device, values=values)
    raise KeyError(f"unknown workload {name!r}")


def skewed_lengths(gen: torch.Generator, n: int, median: int = 512, sigma: float = 1.0,
                   longest: int = 131072, n_single: int = 64):
    """Lognormal lengths (median `median`, log-sd `sigma`) rounded and clipped
    to [1, longest]; one random sequence gets `longest` tokens and `n_single`
    others get one token."""
    z = torch.randn(n, generator=gen, dtype=torch.float64)
    lens = torch.clamp(torch.round(median * torch.exp(sigma * z)), 1, longest).to(torch.int64)
    order = torch.randperm(n, generator=gen)
    lens[order[0]] = longest
    lens[order[1:1 + n_single]] = 1
    return lens.tolist()


NAMES = tuple(SEEDS)

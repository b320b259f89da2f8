"""Plain fp64 CPU oracle for paged-attention decode and the paged cache write.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module. The product path (the HIP library and its
Python binding) never calls it and shares no code with it.

What is computed, and where it comes from:

* Paging. The KV cache is cut into fixed 16-token blocks that a per-sequence
  block table maps to physical blocks, like pages of virtual memory
  ("从零手写 vLLM 核心：mini-vllm 项目深度解析", section "2. 分页KV缓存（PagedAttention）";
  micro-vLLM wiki, the `CacheConfig(block_size=16)` example in its API section).
  K and V live in separate pools, block dimension before the KV-head dimension
  (mini-vllm write-up, "关键工程决策", item 3), so one layer's pool is
  `[num_blocks, block_size, num_kv_heads, head_dim]`.
* Each sequence carries its own cache length (mini-vllm write-up,
  "关键工程决策", item 1); token t of sequence s is at physical block
  `block_tables[s][t // block_size]`, offset `t % block_size`.
* Decode: every running sequence contributes one query token that attends over
  all `context_lens[s]` cached tokens (the write-up's "关键工程决策", item 2:
  steady state is one batched pure-decode step). The result is exact softmax
  attention: gather the sequence's blocks through its table, then
  `out = softmax(scale * q K^T) V` per query head, in float64.
* GQA grouping (not named by the pages; the plainest reading that matches the
  Hugging Face grouping the write-up's parity tests are anchored to, section
  "HF一致性作为正确性锚点"): query head j reads KV head `j // (Hq // Hkv)`.
* Several new tokens per sequence (multi-query): the target model of
  speculative decoding scores the last accepted token and K draft tokens in
  one forward pass ("从零手写 vLLM 核心：mini-vllm 项目深度解析", section
  "推测解码原理"; its "工程启示" section notes the KV-rollback machinery this
  needs), and a prefill chunk appended to a cached prefix is the same shape.
  The n new tokens of a sequence are the last n of its `context_lens[s]`
  cached tokens (their K/V rows are in the pools), and new token i, at
  position L - n + i, attends causally over positions 0..L - n + i: exact
  softmax attention over that prefix, in float64.
* Prefill: a new prompt's tokens attend causally among themselves, the step
  before decode (mini-vllm write-up, section "1. 连续批处理": the scheduler
  mixes prefill of new requests with decode of running ones; "关键工程决策"
  item 2: one forward pass per admitted request). Token t of a prompt attends
  over its tokens 0..t, reading the prompt's own K/V rows.
* Cache write: new token i's K/V row goes to flat slot `slot_mapping[i]`,
  i.e. block `slot // block_size`, offset `slot % block_size`; negative slots
  are padding and are skipped. This is a raw copy, so it is bit-exact.

Storage formats: fp16 and bf16 tensors arrive as their raw 16-bit patterns
(numpy uint16) and are widened to float64 exactly here.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK_SIZE = 16

__all__ = [
    "BLOCK_SIZE",
    "widen",
    "cache_write",
    "gather_sequence",
    "paged_decode",
    "paged_decode_partitioned",
    "paged_multi_query",
    "prefill_attention",
    "round_to_storage",
]


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of raw fp16/bf16 bit patterns (uint16) to float64.

    fp16 goes through numpy's IEEE half type. bf16 is the upper half of an IEEE
    single, so shifting the pattern left by 16 bits gives the float32 with the
    same value, which widens exactly to float64.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError(f"expected raw uint16 bit patterns, got {bits.dtype}")
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to fp16/bf16 (round to nearest, ties to even) and
    return the raw uint16 patterns. Used only to report how far a result is
    from the best representable answer; parity itself compares against the
    unrounded float64 output."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        f = x.astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        # ties-to-even on the 16 dropped bits; NaN stays a quiet NaN
        lsb = (u >> np.uint64(16)) & np.uint64(1)
        r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
        r = np.where(np.isnan(f), np.uint64(0x7FC0), r)
        return r.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def cache_write(k_cache: np.ndarray, v_cache: np.ndarray, key: np.ndarray, value: np.ndarray,
                slot_mapping: np.ndarray, block_size: int = BLOCK_SIZE):
    """Return copies of the two pools with each new row copied into its slot.

    Pools are `[num_blocks, block_size, num_kv_heads, head_dim]`; `key` and
    `value` are `[num_tokens, num_kv_heads, head_dim]`; all of them raw uint16.
    Row i lands at block `slot // block_size`, offset `slot % block_size`
    (flat slot numbering over fixed-size blocks); `slot < 0` means "no write".
    """
    k_new = np.array(k_cache, copy=True)
    v_new = np.array(v_cache, copy=True)
    num_blocks = k_new.shape[0]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        if blk >= num_blocks:
            raise IndexError(f"slot {slot} lies past the pool ({num_blocks} blocks)")
        k_new[blk, off] = key[i]
        v_new[blk, off] = value[i]
    return k_new, v_new


def gather_sequence(cache: np.ndarray, table_row: np.ndarray, length: int,
                    block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Logical `[length, num_kv_heads, head_dim]` view of one sequence's cache:
    its first ceil(length / block_size) physical blocks, in table order, with
    the unused tail of the last block dropped."""
    nblk = -(-length // block_size)
    ids = np.asarray(table_row[:nblk], dtype=np.int64)
    rows = cache[ids]  # [nblk, block_size, Hkv, D]
    return rows.reshape(nblk * block_size, *cache.shape[2:])[:length]


def _check_shapes(q, k_cache, v_cache, block_tables, context_lens, block_size):
    S, Hq, D = q.shape
    NB, BS, Hkv, D2 = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache shapes differ")
    if BS != block_size or D2 != D:
        raise ValueError("pool layout does not match q / block_size")
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables / context_lens do not match num_seqs")
    return S, Hq, Hkv, D


def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 dtype: str, block_size: int = BLOCK_SIZE, return_weights: bool = False):
    """Exact decode attention in float64.

    q: `[S, Hq, D]` raw bits; pools: `[NB, block_size, Hkv, D]` raw bits;
    block_tables: int `[S, max_blocks]`; context_lens: int `[S]`.
    Returns float64 `[S, Hq, D]` (and, if asked, the list of per-sequence
    softmax weights `[Hq, L_s]`). A sequence with no context yields zeros.
    """
    block_tables = np.asarray(block_tables)
    context_lens = np.asarray(context_lens)
    S, Hq, Hkv, D = _check_shapes(q, k_cache, v_cache, block_tables, context_lens, block_size)
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    weights = []
    for s in range(S):
        length = int(context_lens[s])
        if length <= 0:
            weights.append(np.zeros((Hq, 0)))
            continue
        ks = widen(gather_sequence(k_cache, block_tables[s], length, block_size), dtype)
        vs = widen(gather_sequence(v_cache, block_tables[s], length, block_size), dtype)
        w_s = np.empty((Hq, length))
        for j in range(Hq):
            h = j // group
            z = scale * (ks[:, h, :] @ qf[s, j])
            z = z - z.max()
            e = np.exp(z)
            w = e / e.sum()
            w_s[j] = w
            out[s, j] = w @ vs[:, h, :]
        weights.append(w_s)
    if return_weights:
        return out, weights
    return out


def paged_decode_partitioned(q, k_cache, v_cache, block_tables, context_lens, scale: float,
                             dtype: str, partition_tokens: int, block_size: int = BLOCK_SIZE):
    """The same attention computed the split-context way, in float64.

    Each sequence's context is cut into partitions of `partition_tokens`
    tokens. Partition p yields its own maximum logit m_p, its softmax
    denominator l_p = sum exp(z - m_p) and its normalised output
    o_p = sum exp(z - m_p) v / l_p. The partials are merged with the
    log-sum-exp rule: M = max_p m_p, w_p = l_p exp(m_p - M),
    out = sum_p w_p o_p / sum_p w_p, which equals exact softmax attention in
    real arithmetic (the merge used by FlashAttention, Dao et al. 2022).
    """
    if partition_tokens <= 0 or partition_tokens % block_size:
        raise ValueError("partition_tokens must be a positive multiple of block_size")
    block_tables = np.asarray(block_tables)
    context_lens = np.asarray(context_lens)
    S, Hq, Hkv, D = _check_shapes(q, k_cache, v_cache, block_tables, context_lens, block_size)
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        length = int(context_lens[s])
        if length <= 0:
            continue
        ks = widen(gather_sequence(k_cache, block_tables[s], length, block_size), dtype)
        vs = widen(gather_sequence(v_cache, block_tables[s], length, block_size), dtype)
        nparts = -(-length // partition_tokens)
        for j in range(Hq):
            h = j // group
            ms, ls, os_ = [], [], []
            for p in range(nparts):
                lo, hi = p * partition_tokens, min((p + 1) * partition_tokens, length)
                z = scale * (ks[lo:hi, h, :] @ qf[s, j])
                m = z.max()
                e = np.exp(z - m)
                l = e.sum()
                ms.append(m)
                ls.append(l)
                os_.append((e @ vs[lo:hi, h, :]) / l)
            big_m = max(ms)
            w = np.array([l * math.exp(m - big_m) for m, l in zip(ms, ls)])
            out[s, j] = (w[:, None] * np.array(os_)).sum(axis=0) / w.sum()
    return out


def paged_multi_query(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                      block_tables: np.ndarray, context_lens: np.ndarray,
                      query_start: np.ndarray, scale: float, dtype: str,
                      block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Exact causal attention of several new query tokens per sequence, float64.

    Sequence s owns query rows query_start[s] .. query_start[s+1]-1 of q
    (`[T, Hq, D]` raw bits, T = query_start[S]); they are its n_s newest
    tokens, the last n_s of its context_lens[s] = L_s cached tokens. Row
    query_start[s] + i holds the token at position L_s - n_s + i, which
    attends over positions 0 .. L_s - n_s + i. A sequence with n_s = 0 has no
    rows; n_s > L_s is invalid. Returns float64 `[T, Hq, D]`.
    """
    block_tables = np.asarray(block_tables)
    context_lens = np.asarray(context_lens)
    query_start = np.asarray(query_start, dtype=np.int64)
    S = context_lens.shape[0]
    T, Hq, D = q.shape
    NB, BS, Hkv, D2 = k_cache.shape
    if v_cache.shape != k_cache.shape or BS != block_size or D2 != D or Hq % Hkv:
        raise ValueError("pool layout does not match q / block_size / head counts")
    if block_tables.shape[0] != S or query_start.shape[0] != S + 1 or query_start[0] != 0 \
            or query_start[S] != T or np.any(np.diff(query_start) < 0):
        raise ValueError("query_start must run from 0 to T without decreasing, one entry per sequence + 1")
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(S):
        length = int(context_lens[s])
        first, n_new = int(query_start[s]), int(query_start[s + 1] - query_start[s])
        if n_new == 0:
            continue
        if n_new > length:
            raise ValueError(f"sequence {s}: {n_new} new tokens but only {length} in its context")
        ks = widen(gather_sequence(k_cache, block_tables[s], length, block_size), dtype)
        vs = widen(gather_sequence(v_cache, block_tables[s], length, block_size), dtype)
        for i in range(n_new):
            row = first + i
            visible = length - n_new + i + 1      # positions 0 .. L - n + i
            for j in range(Hq):
                h = j // group
                z = scale * (ks[:visible, h, :] @ qf[row, j])
                z = z - z.max()
                e = np.exp(z)
                out[row, j] = (e / e.sum()) @ vs[:visible, h, :]
    return out


def prefill_attention(q: np.ndarray, key: np.ndarray, value: np.ndarray,
                      cu_seqlens: np.ndarray, scale: float, dtype: str) -> np.ndarray:
    """Exact causal self-attention of new prompts, in float64.

    q: `[T, Hq, D]`, key/value: `[T, Hkv, D]` raw bits, all prompts packed;
    prompt s owns rows cu_seqlens[s] .. cu_seqlens[s+1]-1. Token t of a
    prompt (row cu_seqlens[s] + t) attends over the prompt's rows 0..t, query
    head j reading KV head j // (Hq / Hkv). Returns float64 `[T, Hq, D]`.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T, Hq, D = q.shape
    if key.shape != value.shape or key.shape[0] != T or key.shape[2] != D or Hq % key.shape[1]:
        raise ValueError("q / key / value shapes do not match")
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must run from 0 to T without decreasing")
    group = Hq // key.shape[1]
    qf, kf, vf = widen(q, dtype), widen(key, dtype), widen(value, dtype)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        for t in range(hi - lo):
            row = lo + t
            for j in range(Hq):
                h = j // group
                z = scale * (kf[lo:row + 1, h, :] @ qf[row, j])
                z = z - z.max()
                e = np.exp(z)
                out[row, j] = (e / e.sum()) @ vf[lo:row + 1, h, :]
    return out


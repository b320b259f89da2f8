"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each `pin_*` takes an oracle-like module `o` (attributes `paged_decode`,
`paged_decode_partitioned`, `paged_multi_query`, `cache_write`, `widen`) and
raises AssertionError
(or any exception) when the oracle disagrees with:

* hand-derived closed-form cases (tests/golden/closed_form_decode.json,
  tests/golden/cache_write_small.json),
* pure-Python brute force over contiguous K/V (tests/bruteforce.py),
* invariants of softmax attention over a paged cache: relabelling physical
  blocks, sharing prefix blocks vs copying them, a one-token context, q = 0,
  constant V rows, a constant shift of every logit, GQA vs expanded MHA,
* a library routine: torch's scaled_dot_product_attention in float64 on CPU,
* the exact 16-bit patterns of known fp16/bf16 values.

The same functions run against deliberately broken copies of the oracle in
test_oracle_mutants.py, which shows that every planted mistake trips a pin.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from bruteforce import attend_contiguous

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
BS = 16
NAN = {"f16": 0x7E00, "bf16": 0x7FC0}


# ------------------------------------------------------------------ helpers

def bits_of(values, dtype):
    """Exact 16-bit patterns of values that the storage type represents exactly."""
    x = np.asarray(values, dtype=np.float64)
    if dtype == "f16":
        h = x.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), x, equal_nan=True), "value not exact in fp16"
        return h.view(np.uint16)
    f = x.astype(np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0) or np.isnan(x).any(), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def random_dyadic(rng, shape, lo=-24, hi=24, denom=8.0):
    """Random values k/denom, exactly representable in both fp16 and bf16."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64) / denom


def build_paged(rng, k_seq, v_seq, num_blocks, dtype, poison=True):
    """Place contiguous per-sequence K/V ([L, Hkv, D] float64 lists) into pools
    through random distinct physical blocks. Returns bits pools and tables."""
    hkv, d = k_seq[0].shape[1:]
    need = [-(-len(k) // BS) for k in k_seq]
    assert sum(need) <= num_blocks
    perm = rng.permutation(num_blocks)
    fill = NAN[dtype] if poison else 0
    kp = np.full((num_blocks, BS, hkv, d), fill, dtype=np.uint16)
    vp = np.full((num_blocks, BS, hkv, d), fill, dtype=np.uint16)
    tables = np.full((len(k_seq), max(need)), -1, dtype=np.int32)
    cur = 0
    for s, (ks, vs) in enumerate(zip(k_seq, v_seq)):
        for b in range(need[s]):
            tables[s, b] = perm[cur]
            cur += 1
        for t in range(len(ks)):
            kp[tables[s, t // BS], t % BS] = bits_of(ks[t], dtype)
            vp[tables[s, t // BS], t % BS] = bits_of(vs[t], dtype)
    return kp, vp, tables


def random_case(rng, dtype, lens, hq, hkv, d, extra_blocks=3, poison=True):
    k_seq = [random_dyadic(rng, (L, hkv, d)) for L in lens]
    v_seq = [random_dyadic(rng, (L, hkv, d)) for L in lens]
    q = random_dyadic(rng, (len(lens), hq, d))
    nb = sum(-(-L // BS) for L in lens) + extra_blocks
    kp, vp, tables = build_paged(rng, k_seq, v_seq, nb, dtype, poison)
    return dict(q=bits_of(q, dtype), qf=q, k_seq=k_seq, v_seq=v_seq, kp=kp, vp=vp,
                tables=tables, lens=np.array(lens, dtype=np.int32), dtype=dtype)


def run(o, c, scale, **kw):
    return o.paged_decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], scale, c["dtype"], **kw)


def load_golden_case(case):
    dtype = case["dtype"]
    nb, hq, hkv, d = case["num_blocks"], case["num_q_heads"], case["num_kv_heads"], case["head_dim"]
    kp = np.full((nb, BS, hkv, d), NAN[dtype], dtype=np.uint16)
    vp = np.full((nb, BS, hkv, d), NAN[dtype], dtype=np.uint16)
    for r in case["rows"]:
        kp[r["block"], r["offset"]] = bits_of(r["k"], dtype)
        vp[r["block"], r["offset"]] = bits_of(r["v"], dtype)
    q = bits_of(case["q"], dtype)
    scale = eval(case["scale"], {"__builtins__": {}}, {"log": math.log, "sqrt": math.sqrt})
    expected = np.array([[[float(Fraction(x)) for x in row] for row in seq]
                         for seq in case["expected"]])
    return q, kp, vp, np.array(case["block_tables"], dtype=np.int32), \
        np.array(case["context_lens"], dtype=np.int32), float(scale), dtype, expected


# --------------------------------------------------------------------- pins

def pin_widen_known_patterns(o):
    f16 = {0x3C00: 1.0, 0xC000: -2.0, 0x3555: 0.333251953125, 0x0001: 2.0 ** -24,
           0x7BFF: 65504.0, 0x8000: -0.0}
    bf16 = {0x3F80: 1.0, 0xC000: -2.0, 0x4049: 3.140625, 0x0001: 2.0 ** -133,
            0x7F7F: 3.3895313892515355e38, 0x3EAB: 0.333984375}
    for table, dt in ((f16, "f16"), (bf16, "bf16")):
        got = o.widen(np.array(list(table), dtype=np.uint16), dt)
        assert np.array_equal(got, np.array(list(table.values()))), (dt, got)


def pin_golden_decode(o):
    with open(os.path.join(GOLDEN, "closed_form_decode.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        q, kp, vp, bt, cl, scale, dtype, expected = load_golden_case(case)
        got = o.paged_decode(q, kp, vp, bt, cl, scale, dtype)
        assert np.all(np.isfinite(got)), case["name"]
        assert np.allclose(got, expected, rtol=0, atol=1e-12), (case["name"], got, expected)


def pin_golden_cache_write(o):
    with open(os.path.join(GOLDEN, "cache_write_small.json")) as f:
        c = json.load(f)
    dt = c["dtype"]
    shape = (c["num_blocks"], BS, c["num_kv_heads"], c["head_dim"])
    kp = np.zeros(shape, dtype=np.uint16)
    vp = np.zeros(shape, dtype=np.uint16)
    k2, v2 = o.cache_write(kp, vp, bits_of(c["key"], dt), bits_of(c["value"], dt),
                           np.array(c["slot_mapping"], dtype=np.int32))
    ek, ev = np.zeros(shape, dtype=np.uint16), np.zeros(shape, dtype=np.uint16)
    for r in c["expected_rows"]:
        ek[r["block"], r["offset"]] = bits_of(r["k"], dt)
        ev[r["block"], r["offset"]] = bits_of(r["v"], dt)
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)
    assert not np.shares_memory(k2, kp) and np.all(kp == 0), "inputs must not be modified"


def pin_cache_write_negative_slot_noop(o):
    rng = np.random.default_rng(11)
    kp = rng.integers(0, 1 << 16, size=(4, BS, 2, 8), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(4, BS, 2, 8), dtype=np.uint16)
    rows = rng.integers(0, 1 << 16, size=(3, 2, 8), dtype=np.uint16)
    k2, v2 = o.cache_write(kp, vp, rows, rows, np.array([-1, -7, -16], dtype=np.int32))
    assert np.array_equal(k2, kp) and np.array_equal(v2, vp)


def pin_cache_write_random_bruteforce(o):
    rng = np.random.default_rng(12)
    nb, hkv, d = 6, 2, 8
    kp = rng.integers(0, 1 << 16, size=(nb, BS, hkv, d), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(nb, BS, hkv, d), dtype=np.uint16)
    slots = rng.permutation(nb * BS)[:20].astype(np.int32)
    slots[::5] = -1
    key = rng.integers(0, 1 << 16, size=(20, hkv, d), dtype=np.uint16)
    val = rng.integers(0, 1 << 16, size=(20, hkv, d), dtype=np.uint16)
    k2, v2 = o.cache_write(kp, vp, key, val, slots)
    flat_k, flat_v = kp.reshape(nb * BS, hkv, d).copy(), vp.reshape(nb * BS, hkv, d).copy()
    for i, s in enumerate(slots):
        if s >= 0:
            flat_k[s], flat_v[s] = key[i], val[i]
    assert np.array_equal(k2.reshape(nb * BS, hkv, d), flat_k)
    assert np.array_equal(v2.reshape(nb * BS, hkv, d), flat_v)


def pin_bruteforce(o):
    rng = np.random.default_rng(1)
    for dtype, lens, hq, hkv, d in (("f16", [1, 17, 32, 45], 4, 2, 8),
                                    ("bf16", [16, 3, 33], 8, 2, 4),
                                    ("f16", [5, 20], 3, 3, 6),
                                    ("bf16", [49], 8, 1, 4)):
        c = random_case(rng, dtype, lens, hq, hkv, d)
        scale = 0.37
        got = run(o, c, scale)
        for s in range(len(lens)):
            ref = attend_contiguous(c["qf"][s].tolist(), c["k_seq"][s].tolist(),
                                    c["v_seq"][s].tolist(), scale, hkv)
            assert np.allclose(got[s], np.array(ref), rtol=0, atol=1e-12), (dtype, lens, s)


def pin_permutation_invariance(o):
    rng = np.random.default_rng(2)
    c = random_case(rng, "bf16", [7, 16, 40, 1], 4, 2, 8, extra_blocks=5)
    ref = run(o, c, 0.5)
    nb = c["kp"].shape[0]
    pi = rng.permutation(nb)          # physical block b moves to pi[b]
    kp2, vp2 = np.empty_like(c["kp"]), np.empty_like(c["vp"])
    kp2[pi], vp2[pi] = c["kp"], c["vp"]
    t2 = np.where(c["tables"] >= 0, pi[np.maximum(c["tables"], 0)], -1).astype(np.int32)
    got = o.paged_decode(c["q"], kp2, vp2, t2, c["lens"], 0.5, "bf16")
    assert np.array_equal(got, ref)


def pin_single_token_returns_v(o):
    rng = np.random.default_rng(3)
    for dtype in ("f16", "bf16"):
        c = random_case(rng, dtype, [1, 1, 1], 4, 2, 8)
        got = run(o, c, 3.0)
        for s in range(3):
            for j in range(4):
                assert np.array_equal(got[s, j], c["v_seq"][s][0, j // 2]), (dtype, s, j)


def pin_weights_sum_to_one(o):
    rng = np.random.default_rng(4)
    c = random_case(rng, "f16", [2, 31, 64], 4, 4, 8)
    _, weights = run(o, c, 0.8, return_weights=True)
    for s, w in enumerate(weights):
        assert w.shape == (4, c["lens"][s])
        assert np.all(w >= 0)
        assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def pin_zero_query_is_mean(o):
    rng = np.random.default_rng(5)
    c = random_case(rng, "bf16", [1, 9, 50], 2, 1, 4)
    c["q"] = bits_of(np.zeros_like(c["qf"]), "bf16")
    got = run(o, c, 1.0)
    for s in range(3):
        vs = c["v_seq"][s]
        mean = [math.fsum(vs[:, 0, i]) / len(vs) for i in range(4)]
        for j in range(2):
            assert np.allclose(got[s, j], mean, rtol=0, atol=1e-12)


def pin_constant_v_rows(o):
    rng = np.random.default_rng(6)
    c = random_case(rng, "f16", [23, 4], 4, 2, 8)
    row = random_dyadic(rng, (2, 8))
    for s in range(2):
        c["v_seq"][s][:] = row
    kp, vp, tables = build_paged(np.random.default_rng(60), c["k_seq"], c["v_seq"],
                                 c["kp"].shape[0], "f16")
    got = o.paged_decode(c["q"], kp, vp, tables, c["lens"], 0.9, "f16")
    for s in range(2):
        for j in range(4):
            assert np.allclose(got[s, j], row[j // 2], rtol=0, atol=1e-12)


def pin_logit_shift_invariance(o):
    """Adding the same vector u to every K row adds q.u * scale to every logit
    of a head, which softmax ignores."""
    rng = np.random.default_rng(7)
    lens = [18, 5]
    k_seq = [random_dyadic(rng, (L, 2, 8), -8, 8, 4.0) for L in lens]
    v_seq = [random_dyadic(rng, (L, 2, 8)) for L in lens]
    q = random_dyadic(rng, (2, 4, 8), -8, 8, 4.0)
    u = rng.integers(-3, 4, size=(2, 8)).astype(np.float64)
    k_shift = [k + u for k in k_seq]
    nb = sum(-(-L // BS) for L in lens) + 1
    kp, vp, tb = build_paged(np.random.default_rng(70), k_seq, v_seq, nb, "f16")
    kp2, vp2, tb2 = build_paged(np.random.default_rng(71), k_shift, v_seq, nb, "f16")
    ln = np.array(lens, dtype=np.int32)
    a = o.paged_decode(bits_of(q, "f16"), kp, vp, tb, ln, 0.3, "f16")
    b = o.paged_decode(bits_of(q, "f16"), kp2, vp2, tb2, ln, 0.3, "f16")
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def pin_shared_prefix_equals_copies(o):
    rng = np.random.default_rng(8)
    hkv, d, nshared = 2, 8, 2
    prefix_k = random_dyadic(rng, (nshared * BS, hkv, d))
    prefix_v = random_dyadic(rng, (nshared * BS, hkv, d))
    tails = [random_dyadic(rng, (n, hkv, d)) for n in (5, 16, 1)]
    tails_v = [random_dyadic(rng, (n, hkv, d)) for n in (5, 16, 1)]
    k_seq = [np.concatenate([prefix_k, t]) for t in tails]
    v_seq = [np.concatenate([prefix_v, t]) for t in tails_v]
    lens = np.array([len(k) for k in k_seq], dtype=np.int32)
    q = bits_of(random_dyadic(rng, (3, 4, d)), "bf16")
    # copied: every sequence owns its blocks
    kp, vp, tb = build_paged(np.random.default_rng(80), k_seq, v_seq, 16, "bf16")
    copied = o.paged_decode(q, kp, vp, tb, lens, 0.7, "bf16")
    # shared: one physical copy of the prefix blocks referenced by all tables
    kp2 = np.full_like(kp, NAN["bf16"])
    vp2 = np.full_like(vp, NAN["bf16"])
    tb2 = np.full_like(tb, -1)
    for b in range(nshared):
        kp2[b] = kp[tb[0, b]]
        vp2[b] = vp[tb[0, b]]
    nxt = nshared
    for s in range(3):
        tb2[s, :nshared] = np.arange(nshared)
        for b in range(nshared, -(-int(lens[s]) // BS)):
            kp2[nxt], vp2[nxt] = kp[tb[s, b]], vp[tb[s, b]]
            tb2[s, b] = nxt
            nxt += 1
    shared = o.paged_decode(q, kp2, vp2, tb2, lens, 0.7, "bf16")
    assert np.array_equal(shared, copied)


def pin_gqa_equals_expanded_mha(o):
    rng = np.random.default_rng(9)
    c = random_case(rng, "f16", [20, 3], 8, 2, 8)
    ref = run(o, c, 0.6)
    k_exp = [np.repeat(k, 4, axis=1) for k in c["k_seq"]]
    v_exp = [np.repeat(v, 4, axis=1) for v in c["v_seq"]]
    kp, vp, tb = build_paged(np.random.default_rng(90), k_exp, v_exp, c["kp"].shape[0], "f16")
    got = o.paged_decode(c["q"], kp, vp, tb, c["lens"], 0.6, "f16")
    assert np.array_equal(got, ref)


def pin_torch_sdpa(o):
    import torch
    rng = np.random.default_rng(10)
    c = random_case(rng, "bf16", [37, 1, 16], 8, 2, 16)
    scale = 0.25
    got = run(o, c, scale)
    for s in range(3):
        k = torch.tensor(np.repeat(c["k_seq"][s], 4, axis=1)).permute(1, 0, 2)  # [Hq, L, D]
        v = torch.tensor(np.repeat(c["v_seq"][s], 4, axis=1)).permute(1, 0, 2)
        q = torch.tensor(c["qf"][s])[:, None, :]                                  # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)[:, 0]
        assert np.allclose(got[s], ref.numpy(), rtol=0, atol=1e-12)


def pin_partitioned_merge(o):
    rng = np.random.default_rng(13)
    c = random_case(rng, "f16", [1, 16, 47, 100, 129], 4, 2, 8)
    exact = run(o, c, 0.9)
    for p in (16, 32, 48, 128, 256):
        got = o.paged_decode_partitioned(c["q"], c["kp"], c["vp"], c["tables"], c["lens"],
                                         0.9, "f16", p)
        assert np.allclose(got, exact, rtol=0, atol=1e-12), p


def pin_large_logits_finite(o):
    rng = np.random.default_rng(14)
    c = random_case(rng, "bf16", [40, 3], 2, 1, 8)
    got = run(o, c, 400.0)   # logits span thousands: no overflow allowed
    assert np.all(np.isfinite(got))
    for s in range(2):
        ref = attend_contiguous(c["qf"][s].tolist(), c["k_seq"][s].tolist(),
                                c["v_seq"][s].tolist(), 400.0, 1)
        assert np.allclose(got[s], np.array(ref), rtol=0, atol=1e-12)


# ------------------------------------------- several new tokens per sequence

def mq_case(rng, dtype, lens, news, hq, hkv, d, extra_blocks=3):
    """A paged case plus query rows for `news[s]` new tokens per sequence."""
    c = random_case(rng, dtype, lens, hq, hkv, d, extra_blocks)
    qf = random_dyadic(rng, (sum(news), hq, d))
    c.update(mq_qf=qf, mq_q=bits_of(qf, dtype), news=list(news),
             qstart=np.concatenate([[0], np.cumsum(news)]).astype(np.int32))
    return c


def run_mq(o, c, scale):
    return o.paged_multi_query(c["mq_q"], c["kp"], c["vp"], c["tables"], c["lens"], c["qstart"],
                               scale, c["dtype"])


def mq_rows(c):
    """(sequence, new-token index, q row, visible prefix length) of every row."""
    for s, n in enumerate(c["news"]):
        for i in range(n):
            yield s, i, int(c["qstart"][s]) + i, int(c["lens"][s]) - n + i + 1


def pin_mq_bruteforce(o):
    rng = np.random.default_rng(20)
    for dtype, lens, news, hq, hkv, d in (("f16", [1, 17, 40, 9, 33], [1, 5, 3, 0, 33], 4, 2, 8),
                                          ("bf16", [16, 30], [16, 2], 8, 1, 4)):
        c = mq_case(rng, dtype, lens, news, hq, hkv, d)
        got = run_mq(o, c, 0.41)
        assert got.shape == (sum(news), hq, d)
        for s, i, row, vis in mq_rows(c):
            ref = attend_contiguous(c["mq_qf"][row].tolist(), c["k_seq"][s][:vis].tolist(),
                                    c["v_seq"][s][:vis].tolist(), 0.41, hkv)
            assert np.allclose(got[row], np.array(ref), rtol=0, atol=1e-12), (dtype, s, i)


def pin_mq_torch_sdpa_causal(o):
    """torch's attention with an explicit mask over contiguous K/V: new token i
    of a sequence with L cached tokens, n of them new, sees t <= L - n + i."""
    import torch
    rng = np.random.default_rng(21)
    lens, news, g = [45, 7, 20], [4, 7, 1], 4
    c = mq_case(rng, "bf16", lens, news, 8, 2, 16)
    got = run_mq(o, c, 0.25)
    for s, (L, n) in enumerate(zip(lens, news)):
        k = torch.tensor(np.repeat(c["k_seq"][s], g, axis=1)).permute(1, 0, 2)   # [Hq, L, D]
        v = torch.tensor(np.repeat(c["v_seq"][s], g, axis=1)).permute(1, 0, 2)
        r0 = int(c["qstart"][s])
        q = torch.tensor(c["mq_qf"][r0:r0 + n]).permute(1, 0, 2)                  # [Hq, n, D]
        mask = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]     # [n, L]
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=0.25)
        assert np.allclose(got[r0:r0 + n], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12), s


def pin_mq_zero_query_is_prefix_mean(o):
    rng = np.random.default_rng(22)
    c = mq_case(rng, "f16", [12, 40], [6, 3], 2, 1, 4)
    c["mq_q"] = bits_of(np.zeros_like(c["mq_qf"]), "f16")
    got = run_mq(o, c, 1.0)
    for s, i, row, vis in mq_rows(c):
        vs = c["v_seq"][s][:vis, 0]
        mean = [math.fsum(vs[:, e]) / vis for e in range(4)]
        for j in range(2):
            assert np.allclose(got[row, j], mean, rtol=0, atol=1e-12), (s, i)


def pin_mq_first_prefill_token_returns_v0(o):
    """A sequence whose whole context is new: its first token sees only itself."""
    rng = np.random.default_rng(23)
    c = mq_case(rng, "bf16", [21, 5], [21, 5], 4, 2, 8)
    got = run_mq(o, c, 2.0)
    for s in range(2):
        row = int(c["qstart"][s])
        for j in range(4):
            assert np.array_equal(got[row, j], c["v_seq"][s][0, j // 2]), (s, j)


def pin_mq_one_new_token_is_decode(o):
    rng = np.random.default_rng(24)
    c = mq_case(rng, "f16", [1, 30, 64, 17], [1, 1, 1, 1], 8, 2, 8)
    got = run_mq(o, c, 0.7)
    ref = o.paged_decode(c["mq_q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.7, "f16")
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


def pin_mq_permutation_invariance(o):
    rng = np.random.default_rng(25)
    c = mq_case(rng, "bf16", [33, 9, 50], [4, 9, 2], 4, 2, 8, extra_blocks=6)
    ref = run_mq(o, c, 0.5)
    pi = rng.permutation(c["kp"].shape[0])
    kp2, vp2 = np.empty_like(c["kp"]), np.empty_like(c["vp"])
    kp2[pi], vp2[pi] = c["kp"], c["vp"]
    t2 = np.where(c["tables"] >= 0, pi[np.maximum(c["tables"], 0)], -1).astype(np.int32)
    got = o.paged_multi_query(c["mq_q"], kp2, vp2, t2, c["lens"], c["qstart"], 0.5, "bf16")
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- prefill

def prefill_case(rng, dtype, lens, hq, hkv, d):
    q = random_dyadic(rng, (sum(lens), hq, d))
    k = random_dyadic(rng, (sum(lens), hkv, d))
    v = random_dyadic(rng, (sum(lens), hkv, d))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(qf=q, kf=k, vf=v, q=bits_of(q, dtype), k=bits_of(k, dtype), v=bits_of(v, dtype),
                cu=cu, lens=list(lens), dtype=dtype)


def run_prefill(o, c, scale):
    return o.prefill_attention(c["q"], c["k"], c["v"], c["cu"], scale, c["dtype"])


def pin_prefill_torch_sdpa_causal(o):
    import torch
    rng = np.random.default_rng(30)
    c = prefill_case(rng, "bf16", [9, 1, 24], 8, 2, 16)
    got = run_prefill(o, c, 0.3)
    for s, n in enumerate(c["lens"]):
        lo = int(c["cu"][s])
        q = torch.tensor(c["qf"][lo:lo + n]).permute(1, 0, 2)                        # [Hq, n, D]
        k = torch.tensor(np.repeat(c["kf"][lo:lo + n], 4, axis=1)).permute(1, 0, 2)
        v = torch.tensor(np.repeat(c["vf"][lo:lo + n], 4, axis=1)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=0.3)
        assert np.allclose(got[lo:lo + n], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12), s


def pin_prefill_bruteforce(o):
    rng = np.random.default_rng(31)
    c = prefill_case(rng, "f16", [5, 17, 2], 4, 2, 8)
    got = run_prefill(o, c, 0.6)
    for s, n in enumerate(c["lens"]):
        lo = int(c["cu"][s])
        for t in range(n):
            ref = attend_contiguous(c["qf"][lo + t].tolist(), c["kf"][lo:lo + t + 1].tolist(),
                                    c["vf"][lo:lo + t + 1].tolist(), 0.6, 2)
            assert np.allclose(got[lo + t], np.array(ref), rtol=0, atol=1e-12), (s, t)


def pin_prefill_first_token_returns_v0(o):
    rng = np.random.default_rng(32)
    c = prefill_case(rng, "bf16", [3, 7], 4, 2, 8)
    got = run_prefill(o, c, 5.0)
    for s in range(2):
        lo = int(c["cu"][s])
        for j in range(4):
            assert np.array_equal(got[lo, j], c["vf"][lo, j // 2]), (s, j)


def pin_prefill_equals_multi_query_all_new(o):
    """A prompt whose rows sit in a paged cache is the multi-query case with
    every token new (n = L): the two definitions must agree."""
    rng = np.random.default_rng(33)
    lens = [12, 33, 1]
    c = prefill_case(rng, "f16", lens, 8, 2, 8)
    got = run_prefill(o, c, 0.45)
    k_seq = [c["kf"][c["cu"][s]:c["cu"][s + 1]] for s in range(3)]
    v_seq = [c["vf"][c["cu"][s]:c["cu"][s + 1]] for s in range(3)]
    kp, vp, tb = build_paged(np.random.default_rng(330), k_seq, v_seq, 8, "f16")
    ref = o.paged_multi_query(c["q"], kp, vp, tb, np.array(lens, dtype=np.int32), c["cu"], 0.45,
                              "f16")
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

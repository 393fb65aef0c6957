"""Pins for the CPU oracle: it is checked against things other than itself.

* brute force in Python floats on tiny inputs (dense, unpaged);
* a library routine (torch's scaled_dot_product_attention on the CPU, fp64);
* the worked examples printed on the pages (tests/golden/page_examples.json);
* closed forms and invariants of softmax attention over a paged cache.

Each pin is a plain function so that ``test_planted_mistakes_are_caught`` can
run the whole set against deliberately broken copies of the oracle (mistakes
planted on the CPU, in the oracle) and check that each mistake fails a pin.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.paged_attention as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")


# --------------------------------------------------------------------------
# Test-side input construction (not oracle code): a dense problem scattered
# into shuffled physical pages of a NaN-filled pool.
# --------------------------------------------------------------------------

def scatter_dense(k_dense, v_dense, block_size, num_blocks, rng, fill=np.nan):
    """k_dense/v_dense: [Hkv, L, D] float32 -> (k_cache, v_cache, table)."""
    hkv, length, d = k_dense.shape
    nb = -(-length // block_size)
    ids = rng.permutation(num_blocks)[:nb]
    kc = np.full((num_blocks, hkv, block_size, d), fill, dtype=np.float32)
    vc = np.full_like(kc, fill)
    for t in range(length):
        kc[ids[t // block_size], :, t % block_size, :] = k_dense[:, t, :]
        vc[ids[t // block_size], :, t % block_size, :] = v_dense[:, t, :]
    return kc, vc, ids.astype(np.int32)


def dense_case(rng, h, hkv, d, length, bs=16, num_blocks=None):
    q = rng.standard_normal((h, d)).astype(np.float32)
    k = rng.standard_normal((hkv, length, d)).astype(np.float32)
    v = rng.standard_normal((hkv, length, d)).astype(np.float32)
    num_blocks = num_blocks or (-(-length // bs) + 5)
    kc, vc, table = scatter_dense(k, v, bs, num_blocks, rng)
    return q, k, v, kc, vc, table


def run_decode(q, kc, vc, table, length, scale):
    out = op.decode(q[None], kc, vc, table[None], np.array([length]), scale, op.F32)
    return out[0]


def brute(q, k, v, scale):
    """Python-float softmax attention of one query; q [D], k/v [L, D]."""
    z = [scale * sum(float(a) * float(b) for a, b in zip(q, row)) for row in k]
    m = max(z)
    e = [math.exp(x - m) for x in z]
    s = sum(e)
    return [sum(e[t] * float(v[t][j]) for t in range(len(e))) / s for j in range(len(q))]


# --------------------------------------------------------------------------
# Pins
# --------------------------------------------------------------------------

def pin_bruteforce():
    rng = np.random.default_rng(11)
    for h, hkv, d, length, bs in [(2, 2, 8, 1, 16), (2, 1, 8, 5, 4), (4, 2, 16, 8, 4),
                                  (3, 3, 4, 7, 2)]:
        q, k, v, kc, vc, table = dense_case(rng, h, hkv, d, length, bs)
        scale = float(np.float32(1 / math.sqrt(d)))
        out = run_decode(q, kc, vc, table, length, scale)
        g = h // hkv
        for hh in range(h):
            ref = brute(q[hh], k[hh // g], v[hh // g], scale)
            assert np.allclose(out[hh], ref, rtol=0, atol=1e-12), (h, hkv, hh)


def pin_sdpa():
    rng = np.random.default_rng(12)
    for h, hkv, d, length, bs in [(4, 4, 64, 100, 16), (8, 2, 32, 77, 16),
                                  (8, 1, 16, 33, 32), (6, 3, 8, 1, 16)]:
        q, k, v, kc, vc, table = dense_case(rng, h, hkv, d, length, bs)
        scale = float(np.float32(0.37))
        out = run_decode(q, kc, vc, table, length, scale)
        g = h // hkv
        kt = torch.from_numpy(k).double().repeat_interleave(g, dim=0)[None]
        vt = torch.from_numpy(v).double().repeat_interleave(g, dim=0)[None]
        qt = torch.from_numpy(q).double()[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
        assert np.allclose(out, ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


def pin_worked_tables():
    golden = json.load(open(GOLDEN))
    for ex in golden["block_table_examples"]:
        bs = ex["block_size"]
        table = np.array(ex["logical_to_physical"], dtype=np.int32)
        length = bs * len(table)
        nb = int(table.max()) + 4
        kc = np.full((nb, 1, bs, 2), np.nan, dtype=np.float32)
        for j, phys in enumerate(table):
            for o in range(bs):
                kc[phys, 0, o, :] = j * bs + o  # marker = logical token index
        got = op.gather_context(kc, table, length)
        assert np.array_equal(got[0, :, 0], np.arange(length, dtype=np.float32))
        # Attention over it: one-hot-like keys pick the logical token 2*bs+3.
        target = 2 * bs + 3
        kk = np.zeros((nb, 1, bs, 2), dtype=np.float32)
        kk[table[target // bs], 0, target % bs, 0] = 1.0
        q = np.array([[60.0, 0.0]], dtype=np.float32)
        out = op.decode(q[None], kk, kc, table[None], np.array([length]), 1.0, op.F32)
        assert abs(out[0, 0, 0] - target) < 1e-6


def pin_block_counts():
    for ex in json.load(open(GOLDEN))["block_count_examples"]:
        assert op.num_required_blocks(ex["tokens"], ex["block_size"]) == ex["blocks"]
    assert op.num_required_blocks(0, 16) == 0
    assert op.num_required_blocks(17, 16) == 2


def pin_kv_bytes():
    ex = json.load(open(GOLDEN))["kv_size_example"]
    head_dim = ex["hidden_size"] // ex["heads"]
    got = op.kv_cache_bytes(ex["layers"], ex["heads"], ex["tokens"], head_dim,
                            ex["itemsize_matching_print"])
    assert got == ex["expected_bytes"]
    assert abs(got / 2**30 - ex["printed_gib_approx"]) / ex["printed_gib_approx"] < 0.03
    # Allocated bytes of a cache pair equal the formula for one layer.
    nb, hkv, bs, d = 13, 4, 16, 64
    kc = np.zeros((nb, hkv, bs, d), dtype=np.float32)
    assert 2 * kc.nbytes == op.kv_cache_bytes(1, hkv, nb * bs, d, 4)
    bf = np.zeros((nb, hkv, bs, d), dtype=np.uint16)
    assert 2 * bf.nbytes == op.kv_cache_bytes(1, hkv, nb * bs, d, 2)


def pin_ctx1_returns_v():
    rng = np.random.default_rng(13)
    q, k, v, kc, vc, table = dense_case(rng, 4, 2, 16, 1)
    out = run_decode(q, kc, vc, table, 1, 0.25)
    for hh in range(4):
        assert np.array_equal(out[hh], v[hh // 2, 0].astype(np.float64))


def pin_weights_sum_to_one():
    rng = np.random.default_rng(14)
    q, k, v, kc, vc, table = dense_case(rng, 4, 4, 32, 50)
    _, w = op.decode(q[None], kc, vc, table[None], np.array([50]), 0.2, op.F32,
                     return_weights=True)
    for key, wh in w.items():
        assert abs(wh.sum() - 1.0) < 1e-12
        assert (wh >= 0).all() and len(wh) == 50


def pin_q_zero_gives_mean():
    rng = np.random.default_rng(15)
    q, k, v, kc, vc, table = dense_case(rng, 2, 2, 16, 37)
    out = run_decode(np.zeros_like(q), kc, vc, table, 37, 0.3)
    assert np.allclose(out, v.astype(np.float64).mean(axis=1), rtol=0, atol=1e-12)


def pin_constant_v():
    rng = np.random.default_rng(16)
    q, k, v, kc, vc, table = dense_case(rng, 2, 2, 16, 29)
    c = rng.standard_normal(16).astype(np.float32)
    v[:] = c
    kc2, vc2, table2 = scatter_dense(k, v, 16, 10, rng)
    out = run_decode(q, kc2, vc2, table2, 29, 0.3)
    assert np.allclose(out, np.broadcast_to(c.astype(np.float64), out.shape), rtol=0, atol=1e-12)


def pin_shift_invariance():
    """K + u leaves softmax unchanged; a large shift would overflow a naive exp."""
    rng = np.random.default_rng(17)
    d = 16
    q, k, v, kc, vc, table = dense_case(rng, 1, 1, d, 40)
    scale = 1.0
    u = (q[0] / np.dot(q[0], q[0]) * 1000.0).astype(np.float32)  # q.u = 1000
    k2 = (k + u[None, None, :]).astype(np.float32)
    kc2, vc2, table2 = scatter_dense(k2, v, 16, 8, rng)
    base = run_decode(q, kc, vc, table, 40, scale)
    shifted = run_decode(q, kc2, vc2, table2, 40, scale)
    assert np.isfinite(shifted).all()
    # fp32 rounding of k + u perturbs scores by ~|u| * 2^-24 per element.
    assert np.allclose(base, shifted, rtol=0, atol=1e-3)


def pin_block_permutation():
    rng = np.random.default_rng(18)
    q, k, v, kc, vc, table = dense_case(rng, 4, 2, 16, 45, num_blocks=12)
    perm = rng.permutation(12)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    a = run_decode(q, kc, vc, table, 45, 0.25)
    b = run_decode(q, kc2, vc2, perm[table].astype(np.int32), 45, 0.25)
    assert np.array_equal(a, b)


def pin_block_size_independent():
    rng = np.random.default_rng(19)
    q = rng.standard_normal((4, 16)).astype(np.float32)
    k = rng.standard_normal((2, 70, 16)).astype(np.float32)
    v = rng.standard_normal((2, 70, 16)).astype(np.float32)
    outs = []
    for bs in (16, 32):
        kc, vc, table = scatter_dense(k, v, bs, 8, rng)
        outs.append(run_decode(q, kc, vc, table, 70, 0.25))
    assert np.allclose(outs[0], outs[1], rtol=0, atol=1e-13)


def pin_gqa_equals_repeated_mha():
    rng = np.random.default_rng(20)
    q, k, v, kc, vc, table = dense_case(rng, 8, 2, 16, 21)
    gqa = run_decode(q, kc, vc, table, 21, 0.25)
    k_rep = np.repeat(k, 4, axis=0)
    v_rep = np.repeat(v, 4, axis=0)
    kc2, vc2, table2 = scatter_dense(k_rep, v_rep, 16, 6, rng)
    mha = run_decode(q, kc2, vc2, table2, 21, 0.25)
    assert np.array_equal(gqa, mha)


def pin_nan_poison_ignored():
    rng = np.random.default_rng(21)
    q, k, v, kc, vc, table = dense_case(rng, 2, 2, 16, 19)  # pool is NaN-filled
    assert np.isnan(kc).any()
    out = run_decode(q, kc, vc, table, 19, 0.25)
    assert np.isfinite(out).all()
    kc0 = np.nan_to_num(kc, nan=0.0)
    vc0 = np.nan_to_num(vc, nan=0.0)
    assert np.array_equal(out, run_decode(q, kc0, vc0, table, 19, 0.25))


def pin_zero_context():
    q = np.ones((1, 3, 8), dtype=np.float32)
    kc = np.full((2, 3, 16, 8), np.nan, dtype=np.float32)
    out = op.decode(q, kc, kc, np.array([[-1]], dtype=np.int32), np.array([0]), 1.0, op.F32)
    assert np.array_equal(out, np.zeros((1, 3, 8)))


def pin_batch_invariance():
    rng = np.random.default_rng(22)
    q1, k1, v1, kc, vc, t1 = dense_case(rng, 2, 2, 8, 30, num_blocks=20)
    q2 = rng.standard_normal((2, 8)).astype(np.float32)
    tables = np.full((2, 2), -1, dtype=np.int32)
    tables[0, :2] = t1
    tables[1, 0] = [b for b in range(20) if b not in t1][0]
    both = op.decode(np.stack([q1, q2]), kc, vc, tables, np.array([30, 5]), 0.3, op.F32)
    alone = run_decode(q1, kc, vc, t1, 30, 0.3)
    assert np.array_equal(both[0], alone)


def pin_widen():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F80, 0xFF80, 0x3EAB], dtype=np.uint16)
    got = op.widen(bits, op.BF16)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0 ** -133
    assert got[3] == np.inf and got[4] == -np.inf
    assert np.isnan(op.widen(np.array([0x7FC0], dtype=np.uint16), op.BF16)).all()
    rng = np.random.default_rng(23)
    x = torch.from_numpy(rng.standard_normal(1000).astype(np.float32)).to(torch.bfloat16)
    ref = x.double().numpy()
    got = op.widen(x.view(torch.int16).numpy().view(np.uint16), op.BF16)
    assert np.array_equal(got, ref)


def pin_reshape_library():
    """Slot writes equal a fancy-index store into the [NB*BS, Hkv, D] view."""
    rng = np.random.default_rng(24)
    nb, hkv, bs, d, t = 9, 3, 16, 8, 20
    kc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    key = rng.standard_normal((t, hkv, d)).astype(np.float32)
    val = rng.standard_normal((t, hkv, d)).astype(np.float32)
    slots = rng.choice(nb * bs, size=t, replace=False).astype(np.int64)
    slots[[3, 7]] = -1
    ref_k, ref_v = kc.copy(), vc.copy()
    keep = slots >= 0
    view_k = ref_k.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)
    view_v = ref_v.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)
    view_k[slots[keep]] = key[keep]
    view_v[slots[keep]] = val[keep]
    ref_k = view_k.reshape(nb, bs, hkv, d).transpose(0, 2, 1, 3)
    ref_v = view_v.reshape(nb, bs, hkv, d).transpose(0, 2, 1, 3)
    op.reshape_and_cache(key, val, kc, vc, slots)
    assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)


def pin_reshape_roundtrip():
    rng = np.random.default_rng(25)
    nb, hkv, bs, d = 6, 2, 32, 4
    kc = np.zeros((nb, hkv, bs, d), dtype=np.uint16)
    vc = np.zeros_like(kc)
    key = rng.integers(0, 2**16, (5, hkv, d), dtype=np.uint16)
    val = rng.integers(0, 2**16, (5, hkv, d), dtype=np.uint16)
    slots = np.array([0, 33, 191, 64, 95], dtype=np.int64)
    op.reshape_and_cache(key, val, kc, vc, slots)
    for i, slot in enumerate(slots):
        assert np.array_equal(kc[slot // bs, :, slot % bs], key[i])
        assert np.array_equal(vc[slot // bs, :, slot % bs], val[i])
    assert kc.astype(bool).sum() == key.astype(bool).sum()


def pin_copy_blocks():
    rng = np.random.default_rng(26)
    kc = rng.integers(0, 2**16, (10, 2, 16, 4), dtype=np.uint16)
    vc = rng.integers(0, 2**16, (10, 2, 16, 4), dtype=np.uint16)
    pairs = np.array([[1, 7], [4, 2], [1, 9]], dtype=np.int64)
    ref_k, ref_v = kc.copy(), vc.copy()
    ref_k[pairs[:, 1]] = kc[pairs[:, 0]]
    ref_v[pairs[:, 1]] = vc[pairs[:, 0]]
    op.copy_blocks(kc, vc, pairs)
    assert np.array_equal(kc, ref_k) and np.array_equal(vc, ref_v)


def pin_e4m3_table():
    """Code values: the format's landmarks and torch's float8_e4m3fn decoding."""
    v = op.e4m3_values()
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # largest finite
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9    # min normal, min subnormal
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x38] == 1.0 and v[0xC0] == -2.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t))
    assert np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])


def pin_e4m3_encode():
    """Encoding: torch's RNE cast in range, round trips, ties, saturation, NaN."""
    rng = np.random.default_rng(31)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-3, 0.05, 1, 30, 200)])
    x = x.astype(np.float32)
    x = x[np.abs(x) < 448.0]  # torch's cast gives NaN past the largest finite value
    got = op.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)
    v = op.e4m3_values()
    finite = [c for c in range(256) if not np.isnan(v[c])]
    assert np.array_equal(op.e4m3_encode(v[finite].astype(np.float32)), np.array(finite, dtype=np.uint8))
    ties = np.array([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9, 400.0, 432.0, -1.0625],
                    dtype=np.float32)
    assert op.e4m3_encode(ties).tolist() == [0x38, 0x3A, 0x00, 0x02, 0x7C, 0x7E, 0xB8]
    big = np.array([448.0, 449.0, 464.0, 1e6, np.inf, -np.inf, -500.0], dtype=np.float32)
    assert op.e4m3_encode(big).tolist() == [0x7E] * 5 + [0xFE, 0xFE]
    assert op.e4m3_encode(np.array([np.nan], dtype=np.float32))[0] & 0x7F == 0x7F


def pin_fp8_reshape_and_decode():
    """An E4M3 cache: stored codes are the encoded scaled rows; decode is the
    softmax attention over the dequantised values (checked against SDPA)."""
    rng = np.random.default_rng(32)
    hkv, h, d, bs, nb, ks, vs = 2, 4, 16, 16, 6, 0.02, 0.03
    kc = np.zeros((nb, hkv, bs, d), dtype=np.uint8)
    vc = np.zeros_like(kc)
    key = torch.from_numpy(rng.standard_normal((20, hkv, d)).astype(np.float32)).to(torch.bfloat16)
    val = torch.from_numpy(rng.standard_normal((20, hkv, d)).astype(np.float32)).to(torch.bfloat16)
    kb = key.view(torch.int16).numpy().view(np.uint16)
    vb = val.view(torch.int16).numpy().view(np.uint16)
    table = np.array([4, 1], dtype=np.int32)
    slots = np.array([table[t // bs] * bs + t % bs for t in range(20)], dtype=np.int64)
    op.reshape_and_cache(kb, vb, kc, vc, slots, src_dtype=op.BF16, k_scale=ks, v_scale=vs)
    inv_k = np.float32(1) / np.float32(ks)
    expect = torch.from_numpy(key.float().numpy() * inv_k).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kc[4, :, 3], expect[3])
    assert np.array_equal(kc[1, :, 2], expect[18])
    q = rng.standard_normal((h, d)).astype(np.float32)
    out = op.decode(q[None], kc, vc, table[None], np.array([20]), 0.25, op.F32,
                    cache_dtype=op.FP8, k_scale=ks, v_scale=vs)[0]
    vals = op.e4m3_values()
    kd = np.stack([vals[kc[table[t // bs], :, t % bs]] for t in range(20)], axis=1) * np.float32(ks)
    vd = np.stack([vals[vc[table[t // bs], :, t % bs]] for t in range(20)], axis=1) * np.float32(vs)
    kt = torch.from_numpy(kd).repeat_interleave(2, dim=0)[None]
    vt = torch.from_numpy(vd).repeat_interleave(2, dim=0)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).double()[None, :, None, :], kt, vt, scale=0.25)
    assert np.allclose(out, ref[0, :, 0].numpy(), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# Several queries per sequence (chunked prefill, speculative verification)
# --------------------------------------------------------------------------

def mq_case(rng, h, hkv, d, seqs, bs=16):
    """seqs: [(context_len, query_len)].  Dense K/V per sequence scattered into
    one shuffled NaN-filled pool; the queries of all sequences stacked."""
    need = [-(-c // bs) for c, _ in seqs]
    nb = sum(need) + 3
    ids = rng.permutation(nb)
    kc = np.full((nb, hkv, bs, d), np.nan, dtype=np.float32)
    vc = np.full_like(kc, np.nan)
    tables = np.full((len(seqs), max(need + [1])), -1, dtype=np.int32)
    dense = []
    at = 0
    for s, (c, _) in enumerate(seqs):
        k = rng.standard_normal((hkv, c, d)).astype(np.float32)
        v = rng.standard_normal((hkv, c, d)).astype(np.float32)
        tables[s, :need[s]] = ids[at:at + need[s]]
        at += need[s]
        for t in range(c):
            kc[tables[s, t // bs], :, t % bs, :] = k[:, t, :]
            vc[tables[s, t // bs], :, t % bs, :] = v[:, t, :]
        dense.append((k, v))
    qs = np.concatenate([[0], np.cumsum([ql for _, ql in seqs])]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), h, d)).astype(np.float32)
    ctx = np.array([c for c, _ in seqs], dtype=np.int32)
    return q, dense, kc, vc, tables, ctx, qs


MQ_CASES = [  # (H, Hkv, D, BS, [(context_len, query_len)])
    (4, 4, 32, 16, [(10, 10), (37, 5), (1, 1), (50, 1), (20, 0)]),
    (8, 2, 16, 16, [(33, 33), (70, 6), (16, 16)]),
    (8, 1, 8, 4, [(9, 3), (5, 5), (12, 12)]),
]


def pin_mq_sdpa():
    """Each chunk equals torch's SDPA (fp64) with the causal mask aligned to the
    end of the context: query i may see tokens j <= L - q_len + i."""
    rng = np.random.default_rng(31)
    for h, hkv, d, bs, seqs in MQ_CASES:
        q, dense, kc, vc, tables, ctx, qs = mq_case(rng, h, hkv, d, seqs, bs)
        scale = float(np.float32(0.3))
        out = op.multi_query(q, kc, vc, tables, ctx, qs, scale, op.F32)
        g = h // hkv
        for s, (c, ql) in enumerate(seqs):
            if ql == 0:
                continue
            k, v = dense[s]
            kt = torch.from_numpy(k).double().repeat_interleave(g, dim=0)[None]
            vt = torch.from_numpy(v).double().repeat_interleave(g, dim=0)[None]
            qt = torch.from_numpy(q[qs[s]:qs[s + 1]]).double().permute(1, 0, 2)[None]
            allowed = torch.arange(c)[None, :] <= (c - ql + torch.arange(ql))[:, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=allowed,
                                                                   scale=scale)
            assert np.allclose(out[qs[s]:qs[s + 1]], ref[0].permute(1, 0, 2).numpy(), rtol=0,
                               atol=1e-12), (h, hkv, s)


def pin_mq_bruteforce():
    rng = np.random.default_rng(32)
    h, hkv, d, bs, seqs = 2, 1, 4, 2, [(5, 3), (3, 3), (4, 1)]
    q, dense, kc, vc, tables, ctx, qs = mq_case(rng, h, hkv, d, seqs, bs)
    scale = float(np.float32(0.5))
    out = op.multi_query(q, kc, vc, tables, ctx, qs, scale, op.F32)
    for s, (c, ql) in enumerate(seqs):
        k, v = dense[s]
        for i in range(ql):
            seen = c - ql + i + 1   # tokens 0 .. c - ql + i
            for hh in range(h):
                ref = brute(q[qs[s] + i, hh], k[0][:seen], v[0][:seen], scale)
                assert np.allclose(out[qs[s] + i, hh], ref, rtol=0, atol=1e-12), (s, i, hh)


def pin_mq_last_query_is_decode():
    """The last query of a chunk sits at position L - 1: plain decode."""
    rng = np.random.default_rng(33)
    for h, hkv, d, bs, seqs in MQ_CASES:
        q, dense, kc, vc, tables, ctx, qs = mq_case(rng, h, hkv, d, seqs, bs)
        out = op.multi_query(q, kc, vc, tables, ctx, qs, 0.25, op.F32)
        for s, (c, ql) in enumerate(seqs):
            if ql == 0:
                continue
            dec = op.decode(q[qs[s + 1] - 1][None], kc, vc, tables[s][None], ctx[s:s + 1], 0.25,
                            op.F32)
            assert np.allclose(out[qs[s + 1] - 1], dec[0], rtol=0, atol=1e-13)


def pin_mq_chunking_invariance():
    """Cutting a chunk in two (the first part at the shorter context) changes
    nothing: the point of chunked prefill."""
    rng = np.random.default_rng(34)
    h, hkv, d, bs = 4, 2, 16, 4
    q, dense, kc, vc, tables, ctx, qs = mq_case(rng, h, hkv, d, [(30, 12)], bs)
    whole = op.multi_query(q, kc, vc, tables, ctx, qs, 0.3, op.F32)
    for cut in (1, 5, 11):
        first = op.multi_query(q[:cut], kc, vc, tables, np.array([30 - 12 + cut], np.int32),
                               np.array([0, cut], np.int32), 0.3, op.F32)
        second = op.multi_query(q[cut:], kc, vc, tables, ctx, np.array([0, 12 - cut], np.int32),
                                0.3, op.F32)
        assert np.allclose(np.concatenate([first, second]), whole, rtol=0, atol=1e-13), cut


def pin_mq_causality():
    """Changing the newest token's K/V changes only the last query's output."""
    rng = np.random.default_rng(35)
    h, hkv, d, bs = 4, 4, 8, 4
    q, dense, kc, vc, tables, ctx, qs = mq_case(rng, h, hkv, d, [(13, 6)], bs)
    before = op.multi_query(q, kc, vc, tables, ctx, qs, 0.3, op.F32)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[tables[0, 12 // bs], :, 12 % bs, :] += 3.0
    vc2[tables[0, 12 // bs], :, 12 % bs, :] -= 2.0
    after = op.multi_query(q, kc2, vc2, tables, ctx, qs, 0.3, op.F32)
    assert np.array_equal(after[:5], before[:5])
    assert not np.allclose(after[5], before[5])


def pin_swap_blocks():
    """Swapping out then in restores the blocks; the rest of both pools is
    untouched; the result equals a fancy-index copy."""
    rng = np.random.default_rng(36)
    dev_k = rng.standard_normal((20, 2, 4, 8)).astype(np.float32)
    dev_v = rng.standard_normal((20, 2, 4, 8)).astype(np.float32)
    host_k = np.full((6, 2, 4, 8), np.nan, dtype=np.float32)
    host_v = host_k.copy()
    out_pairs = np.array([[3, 0], [17, 4], [9, 1]], dtype=np.int64)
    op.swap_blocks(dev_k, dev_v, host_k, host_v, out_pairs)
    assert np.array_equal(host_k[[0, 4, 1]], dev_k[[3, 17, 9]])
    assert np.array_equal(host_v[[0, 4, 1]], dev_v[[3, 17, 9]])
    assert np.isnan(host_k[[2, 3, 5]]).all()
    back_k, back_v = np.zeros_like(dev_k), np.zeros_like(dev_v)
    op.swap_blocks(host_k, host_v, back_k, back_v, np.array([[0, 11], [4, 2], [1, 19]]))
    assert np.array_equal(back_k[[11, 2, 19]], dev_k[[3, 17, 9]])
    assert np.array_equal(back_v[[11, 2, 19]], dev_v[[3, 17, 9]])
    others = [b for b in range(20) if b not in (11, 2, 19)]
    assert not back_k[others].any() and not back_v[others].any()


PINS = [pin_bruteforce, pin_sdpa, pin_worked_tables, pin_block_counts, pin_kv_bytes,
        pin_ctx1_returns_v, pin_weights_sum_to_one, pin_q_zero_gives_mean,
        pin_constant_v, pin_shift_invariance, pin_block_permutation,
        pin_block_size_independent, pin_gqa_equals_repeated_mha,
        pin_nan_poison_ignored, pin_zero_context, pin_batch_invariance, pin_widen,
        pin_reshape_library, pin_reshape_roundtrip, pin_copy_blocks, pin_e4m3_table,
        pin_e4m3_encode, pin_fp8_reshape_and_decode, pin_mq_sdpa, pin_mq_bruteforce,
        pin_mq_last_query_is_decode, pin_mq_chunking_invariance, pin_mq_causality,
        pin_swap_blocks]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# --------------------------------------------------------------------------
# Planted mistakes: each broken oracle must fail at least one pin.
# --------------------------------------------------------------------------

def _interleaved_kv_head(head, num_heads, num_kv_heads):
    return head % num_kv_heads


def _gather_ignoring_table(cache, row, length):
    nb = -(-length // cache.shape[2])
    return np.concatenate([cache[j] for j in range(nb)], axis=1)[:, :length]


def _gather_one_extra(cache, row, length):
    bs = cache.shape[2]
    nb = -(-(length + 1) // bs)
    pages = [cache[int(row[min(j, len(row) - 1)])] for j in range(nb)]
    return np.concatenate(pages, axis=1)[:, :length + 1]


def _softmax_no_max(z):
    w = np.exp(z)
    return w / w.sum()


def _softmax_wrong_norm(z):
    w = np.exp(z - z.max())
    return w / w.max()


def _attend_no_scale(q, k, v, scale):
    w = _softmax_ok(k @ q)
    return w @ v, w


def _attend_transposed(q, k, v, scale):
    w = _softmax_ok(scale * (k @ q))
    return w @ v[:, ::-1], w


def _softmax_ok(z):
    w = np.exp(z - z.max())
    return w / w.sum()


def _widen_bad(x, dtype):
    if dtype == op.BF16:
        return (x.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _reshape_swapped(key, value, kc, vc, slots, **kw):
    bs = kc.shape[2]
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        offset, block = divmod(int(slot), kc.shape[0])
        kc[block % kc.shape[0], :, offset % bs, :] = key[i]
        vc[block % kc.shape[0], :, offset % bs, :] = value[i]


def _copy_k_only(kc, vc, pairs):
    for s, d in np.asarray(pairs).reshape(-1, 2):
        kc[int(d)] = kc[int(s)]


def _e4m3_ties_away(x):
    x = np.asarray(x, dtype=np.float32)
    mags = _E4M3_TRUE_VALUES()[:0x7F]
    out = []
    for v in x.reshape(-1).astype(np.float64):
        sign = 0x80 if np.signbit(v) else 0
        if np.isnan(v):
            out.append(sign | 0x7F)
            continue
        a = min(abs(v), 448.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        out.append(sign | int(best[-1]))   # ties go to the larger magnitude
    return np.array(out, dtype=np.uint8).reshape(x.shape)


def _E4M3_TRUE_VALUES():
    return _ORIG_E4M3_VALUES()


def _e4m3_values_bias8():
    v = _ORIG_E4M3_VALUES().copy()
    return v / 2.0


def _e4m3_no_saturation(x):
    x = np.asarray(x, dtype=np.float32)
    out = _ORIG_E4M3_ENCODE(x)
    over = np.abs(x) > 448.0
    out[over] = 0x7F
    return out


_ORIG_E4M3_VALUES = op.e4m3_values
_ORIG_E4M3_ENCODE = op.e4m3_encode


def _swap_k_only(src_k, src_v, dst_k, dst_v, pairs):
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        dst_k[int(dst)] = src_k[int(src)]


def _swap_pair_reversed(src_k, src_v, dst_k, dst_v, pairs):
    # reads each pair as (dst, src)
    for dst, src in np.asarray(pairs).reshape(-1, 2):
        dst_k[int(dst) % len(dst_k)] = src_k[int(src) % len(src_k)]
        dst_v[int(dst) % len(dst_v)] = src_v[int(src) % len(src_v)]


def _position_plus_one(context_len, query_len, i):
    return context_len - query_len + i + 1


def _position_unmasked(context_len, query_len, i):
    return context_len - 1


def _position_top_left(context_len, query_len, i):
    return i


def _rows_drop_last(query_start, s):
    return int(query_start[s]), max(int(query_start[s]), int(query_start[s + 1]) - 1)

MUTATIONS = {
    "e4m3_ties_away_from_even": ("e4m3_encode", _e4m3_ties_away),
    "e4m3_bias_8": ("e4m3_values", _e4m3_values_bias8),
    "e4m3_overflow_to_nan": ("e4m3_encode", _e4m3_no_saturation),
    "interleaved_kv_head": ("kv_head_for", _interleaved_kv_head),
    "gather_ignores_table": ("gather_context", _gather_ignoring_table),
    "gather_off_by_one": ("gather_context", _gather_one_extra),
    "softmax_without_max": ("softmax", _softmax_no_max),
    "softmax_wrong_normaliser": ("softmax", _softmax_wrong_norm),
    "scale_dropped": ("attend_one", _attend_no_scale),
    "v_dims_reversed": ("attend_one", _attend_transposed),
    "bf16_widen_shift": ("widen", _widen_bad),
    "reshape_block_offset_swapped": ("reshape_and_cache", _reshape_swapped),
    "copy_blocks_k_only": ("copy_blocks", _copy_k_only),
    "mq_causal_mask_one_late": ("query_position", _position_plus_one),
    "mq_no_causal_mask": ("query_position", _position_unmasked),
    "mq_causal_mask_top_left": ("query_position", _position_top_left),
    "mq_query_rows_short": ("query_rows", _rows_drop_last),
    "swap_k_only": ("swap_blocks", _swap_k_only),
    "swap_pair_reversed": ("swap_blocks", _swap_pair_reversed),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(op, attr, bad)
    failed = []
    with np.errstate(all="ignore"):
        for pin in PINS:
            try:
                pin()
            except (AssertionError, ValueError, IndexError, FloatingPointError):
                failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"

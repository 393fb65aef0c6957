"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Reduced-size cases (the oracle finishes them in seconds) are compared element
by element; they span several pages, several partitions and a ragged last
page.  Full-size workloads run in the launch configuration the benchmark uses
and are compared on sampled sequences.  reshape_and_cache and copy_blocks
must match bit for bit; decode within atol 5e-3 + rtol 1e-2 (bf16) or
1e-5 + 1e-5 (fp32) of the fp64 oracle.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_321_amd import binding, workloads as wl

from gpu_helpers import (as_f64, assert_close, bits, gpu_step, on_device, oracle_step,
                         sampled_reference, to_top_of_pool)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny": dict(),
    "llama7b": dict(num_seqs=6, ctx_range=(1, 700), new_tokens=True),
    "llama13b": dict(num_seqs=5, context_len=2048),
    "gqa70b": dict(num_seqs=2, context_len=4100),
    "beam": dict(groups=3, beams=4, prefix_len=64, tail_lo=1, tail_hi=40, cow_fraction=0.5),
}
for _n in ("llama7b", "llama13b", "gqa70b", "beam"):  # the same shapes with an fp8 cache
    SMALL[_n + "_fp8"] = SMALL[_n]


def check_case(x, partition_tokens=0):
    out, t = gpu_step(x, partition_tokens=partition_tokens)
    ref, kc, vc = oracle_step(x)
    assert np.array_equal(bits(t["k_cache"]), bits(kc)), "k_cache differs from the oracle"
    assert np.array_equal(bits(t["v_cache"]), bits(vc)), "v_cache differs from the oracle"
    return assert_close(as_f64(out), ref, x.spec.dtype, x.spec.name)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_workload_small(name):
    x = wl.make_inputs(name, **SMALL[name])
    check_case(x)


@pytest.mark.parametrize("pt", [16, 64, 256, 512])
def test_partitions_llama7b_small(pt):
    x = wl.make_inputs("llama7b", **SMALL["llama7b"])
    check_case(x, partition_tokens=pt)


@pytest.mark.parametrize("pt", [32, 1024])
def test_partitions_gqa_small(pt):
    x = wl.make_inputs("gqa70b", **SMALL["gqa70b"])
    check_case(x, partition_tokens=pt)


@pytest.mark.parametrize("name,kw", [
    ("gqa70b", dict(num_seqs=1, context_len=20000)),
    ("gqa70b_fp8", dict(num_seqs=2, context_len=9000)),
    ("llama13b", dict(num_seqs=2, context_len=5000)),
    ("tiny", dict()),
])
def test_fill_partitions(name, kw):
    """A few long sequences with the batch-shaped partition length
    (PA_PARTITION_FILL): shorter partitions than the fixed ones, same result."""
    x = wl.make_inputs(name, **kw)
    sp = x.spec
    code = {"f32": binding.PA_F32, "bf16": binding.PA_BF16}[sp.dtype]
    ccode = binding.PA_FP8_E4M3 if sp.kv_dtype == "fp8" else code
    args = (x.plan.num_seqs, sp.num_heads, sp.num_kv_heads, sp.head_dim, sp.block_size,
            x.max_context_len, code, ccode)
    pt = binding.pa_decode_partition_tokens(*args, policy=binding.PA_PARTITION_FILL)
    fixed = binding.pa_decode_partition_tokens(*args)
    assert pt <= fixed and (name == "tiny" or pt < fixed)
    check_case(x, partition_tokens=pt)


SHAPES = [
    # (H, Hkv, D, BS, dtype)
    (4, 4, 64, 16, "f32"), (4, 4, 64, 32, "f32"), (4, 2, 128, 16, "f32"), (8, 1, 128, 32, "f32"),
    (8, 8, 64, 16, "bf16"), (8, 4, 64, 32, "bf16"), (16, 4, 128, 16, "bf16"),
    (16, 2, 128, 32, "bf16"), (8, 8, 128, 32, "bf16"),
    # grouped heads on the matrix-core path (bf16, group 2/4/8, both block sizes, both dims)
    (16, 8, 64, 16, "bf16"), (32, 4, 64, 16, "bf16"), (8, 2, 128, 32, "bf16"),
    (16, 8, 128, 16, "bf16"), (64, 8, 128, 32, "bf16"), (32, 8, 128, 16, "bf16"),
]


@pytest.mark.parametrize("h,hkv,d,bs,dtype", SHAPES)
def test_shapes(h, hkv, d, bs, dtype):
    spec = wl.Spec(f"shape{h}x{hkv}x{d}x{bs}{dtype}", h, hkv, d, bs, dtype, seed=h * 100 + d + bs)
    gen = torch.Generator().manual_seed(spec.seed)
    ctx = [0, 1, bs - 1, bs, bs + 1, 3 * bs + 5, 700, 1100]
    plan = wl.uniform_plan(ctx, bs, gen, new_tokens=True)
    x = wl.build_inputs(spec, plan)
    check_case(x)
    check_case(x, partition_tokens=4 * bs)


FP8_SHAPES = [
    # (H, Hkv, D, BS) with a bf16 query and an E4M3 cache
    (8, 8, 128, 16), (8, 8, 64, 32), (16, 8, 128, 32), (16, 4, 64, 16), (32, 4, 128, 16),
    (64, 8, 128, 32), (16, 2, 128, 16),
]


@pytest.mark.parametrize("h,hkv,d,bs", FP8_SHAPES)
def test_shapes_fp8(h, hkv, d, bs):
    spec = wl.Spec(f"fp8shape{h}x{hkv}x{d}x{bs}", h, hkv, d, bs, "bf16", seed=7 * h + d + bs,
                   kv_dtype="fp8", **wl.fp8_scales("fp8"))
    gen = torch.Generator().manual_seed(spec.seed)
    ctx = [0, 1, bs - 1, bs + 1, 3 * bs + 5, 700, 1100]
    plan = wl.uniform_plan(ctx, bs, gen, new_tokens=True)
    x = wl.build_inputs(spec, plan)
    check_case(x)
    check_case(x, partition_tokens=4 * bs)


def _pow2_fp8(name, **kw):
    """A workload of ``name`` whose fp8 caches use the scale 1/64 for K and V
    (special values placed at a chosen code survive the scaling exactly)."""
    base = wl.SPECS[name]
    spec = wl.Spec(base.name + "_pow2", base.num_heads, base.num_kv_heads, base.head_dim,
                   base.block_size, base.dtype, seed=base.seed, q_std=base.q_std,
                   kv_dtype="fp8", k_scale=1.0 / 64, v_scale=1.0 / 64, recipe=base.recipe)
    gen = torch.Generator().manual_seed(spec.seed)
    return wl.build_inputs(spec, wl.make_plan(name, gen, **kw))


def test_fp8_reshape_codes_exact():
    """E4M3 encoding of new rows: ties, subnormals, saturation, NaN, -0, random."""
    import oracle.paged_attention as op
    x = _pow2_fp8("llama13b_fp8", num_seqs=6, context_len=40)
    special = np.array([1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9, 400.0, 432.0, 447.0, 448.0,
                        449.0, 464.0, 1e9, -1e9, 0.0, -0.0, 2.0 ** -12, -(2.0 ** -7),
                        0.015625 * 3.0, 1e-30], dtype=np.float32)
    key = x.key.float().numpy().copy()
    flat = key.reshape(-1)
    flat[: len(special)] = special / np.float32(64.0)  # divided back by the scale in the kernel
    flat[len(special): len(special) + 3] = [np.nan, np.inf, -np.inf]
    x.key = torch.from_numpy(key).to(torch.bfloat16)
    out, t = gpu_step(x)
    ref, kc, vc = oracle_step(x)
    assert np.array_equal(bits(t["k_cache"]), bits(kc))
    assert np.array_equal(bits(t["v_cache"]), bits(vc))
    # The rows really went through the saturating, NaN-preserving encoder.
    slot = int(x.plan.slot_mapping[0])
    row = bits(t["k_cache"])[slot // 16, :, slot % 16].reshape(-1)
    assert row[8] == 0x7E and row[10] == 0x7E and row[11] == 0xFE and row[13] == 0x80
    assert (row[len(special)] & 0x7F) == 0x7F
    nan_row = int(x.plan.new_token_seqs[0])  # its newest token holds the NaN
    others = [r for r in range(x.plan.num_seqs) if r != nan_row]
    assert np.isfinite(as_f64(out)[others]).all()
    assert_close(as_f64(out)[others], ref[others], "bf16", "fp8 rows")


def _encode_rule_witnesses(scale):
    """float32 values whose E4M3 code under x * fl32(1 / scale) differs from
    the code of the correctly rounded quotient fl32(x / scale): a few next to
    every midpoint between two E4M3 magnitudes where the two rules part."""
    import oracle.paged_attention as op
    s32 = np.float32(scale)
    inv = op.e4m3_inverse_scale(scale)
    mags = op.e4m3_values()[:0x7F]
    found = []
    for m in (mags[:-1] + mags[1:]) / 2:
        x0 = np.float32(m * float(s32))
        xs = (np.int32(x0.view(np.int32)) + np.arange(-200, 200, dtype=np.int32)).view(np.float32)
        a = op.e4m3_encode(xs * inv)
        b = op.e4m3_encode((xs / s32).astype(np.float32))
        found.extend(xs[a != b][:2].tolist())
    return np.array(found, dtype=np.float32)


def test_fp8_encode_multiplies_by_rounded_inverse_scale():
    """E4M3 codes of float32 rows at k_scale 0.02 and v_scale 0.03 (distinct,
    not powers of two): bit-exact against the oracle's rule (binary32 product
    with fl32(1 / scale)), with rows placed where a division by the scale, or
    the other cache's scale, would give other codes."""
    import oracle.paged_attention as op
    spec = wl.Spec("fp8_encode_rule", 4, 2, 64, 16, "f32", seed=991, kv_dtype="fp8",
                   **wl.fp8_scales("fp8"))
    gen = torch.Generator().manual_seed(spec.seed)
    plan = wl.uniform_plan([1, 17, 40, 33, 2, 64], 16, gen, new_tokens=True)
    x = wl.build_inputs(spec, plan)
    key, value = x.key.numpy().copy(), x.value.numpy().copy()
    for arr, sc in ((key, x.k_scale), (value, x.v_scale)):
        w = _encode_rule_witnesses(sc)
        assert w.size >= 20, "too few witnesses of the encode rule"
        w = np.concatenate([w, -w])
        n = min(w.size, arr.size)
        arr.reshape(-1)[:n] = w[:n]
    x.key, x.value = torch.from_numpy(key), torch.from_numpy(value)
    t = on_device(x)
    binding.pa_reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"],
                                 t["slot_mapping"], k_scale=x.k_scale, v_scale=x.v_scale)
    torch.cuda.synchronize()
    kc, vc = bits(x.k_cache).copy(), bits(x.v_cache).copy()
    op.reshape_and_cache(key, value, kc, vc, plan.slot_mapping, src_dtype="f32",
                         k_scale=x.k_scale, v_scale=x.v_scale)
    got_k, got_v = bits(t["k_cache"]), bits(t["v_cache"])
    assert np.array_equal(got_k, kc) and np.array_equal(got_v, vc)
    # The same rows under the division rule, and under swapped scales, differ.
    for rule in ("divide", "swap"):
        kd, vd = bits(x.k_cache).copy(), bits(x.v_cache).copy()
        if rule == "divide":
            kq = op.e4m3_encode((key / np.float32(x.k_scale)).astype(np.float32))
            vq = op.e4m3_encode((value / np.float32(x.v_scale)).astype(np.float32))
            op.reshape_and_cache(kq, vq, kd, vd, plan.slot_mapping)
        else:
            op.reshape_and_cache(key, value, kd, vd, plan.slot_mapping, src_dtype="f32",
                                 k_scale=x.v_scale, v_scale=x.k_scale)
        assert not np.array_equal(got_k, kd) and not np.array_equal(got_v, vd), rule


@pytest.mark.parametrize("name", ["gqa70b_fp8", "llama7b_fp8"])
def test_fp8_context_one_every_code_bitwise(name):
    """With one token the output is exactly code value * v_scale (a power of
    two), for every finite E4M3 code, on the matrix-core and vector paths."""
    import oracle.paged_attention as op
    kw = dict(num_seqs=2, context_len=1) if name == "gqa70b_fp8" else \
        dict(num_seqs=2, ctx_range=(1, 1))
    x = _pow2_fp8(name, **kw)
    t = on_device(x)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for s_ in range(x.plan.num_seqs):
        b = int(x.plan.block_tables[s_][0])
        n = x.spec.num_kv_heads * x.spec.head_dim
        pattern = np.resize(np.roll(codes, 37 * s_), n).reshape(x.spec.num_kv_heads, x.spec.head_dim)
        t["v_cache"].view(torch.uint8)[b, :, 0, :] = torch.from_numpy(pattern).cuda()
    out, _ = gpu_step(x, t, copy=False, reshape=False)
    vals = op.e4m3_values()
    g = x.spec.num_heads // x.spec.num_kv_heads
    v = t["v_cache"].view(torch.uint8).cpu().numpy()
    for s_ in range(x.plan.num_seqs):
        b = int(x.plan.block_tables[s_][0])
        want = vals[v[b, :, 0, :]] * x.v_scale                    # exact in float64
        want_bf16 = torch.from_numpy(np.repeat(want, g, axis=0)).float().to(torch.bfloat16)
        assert torch.equal(out[s_].cpu(), want_bf16), s_


def test_zero_context_rows_are_zero():
    x = wl.make_inputs("tiny", context_lens=[0, 5, 0, 40])
    out, _ = gpu_step(x)
    o = as_f64(out)
    assert (o[0] == 0).all() and (o[2] == 0).all()
    check_case(x)


def test_context_one_returns_v_bitwise():
    for name, kw in (("tiny", dict(context_lens=[1, 1, 1, 1])),
                     ("llama13b", dict(num_seqs=3, context_len=1))):
        x = wl.make_inputs(name, **kw)
        out, t = gpu_step(x)
        v = t["v_cache"]
        plan = x.plan
        g = x.spec.num_heads // x.spec.num_kv_heads
        for s in range(plan.num_seqs):
            b = int(plan.block_tables[s][0])
            for h in range(x.spec.num_heads):
                assert torch.equal(out[s, h], v[b, h // g, 0]), (name, s, h)


def test_block_permutation_bitwise():
    x = wl.make_inputs("gqa70b", num_seqs=2, context_len=1500)
    out, t = gpu_step(x, partition_tokens=512)
    nb = x.plan.num_blocks
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(9)).cuda()
    t2 = on_device(x)
    for n in ("k_cache", "v_cache"):
        src = t[n]
        dst = torch.empty_like(src)
        dst[perm] = src
        t2[n] = dst
    bt = t["block_tables"].long()
    t2["block_tables"] = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).int()
    out2, _ = gpu_step(x, t2, partition_tokens=512, copy=False, reshape=False)
    assert torch.equal(out, out2)


def test_batch_invariance_bitwise():
    x = wl.make_inputs("llama7b", **SMALL["llama7b"])
    out, t = gpu_step(x, partition_tokens=256)
    keep = [4, 1]
    t2 = dict(t)
    t2["q"] = t["q"][keep].contiguous()
    t2["block_tables"] = t["block_tables"][keep].contiguous()
    t2["context_lens"] = t["context_lens"][keep].contiguous()
    out2 = torch.empty_like(t2["q"])
    from paged_kv_cache_321_amd import binding
    binding.pa_decode(out2, t2["q"], t["k_cache"], t["v_cache"], t2["block_tables"],
                      t2["context_lens"], x.scale, x.max_context_len, partition_tokens=256)
    torch.cuda.synchronize()
    assert torch.equal(out[keep], out2)


@pytest.mark.parametrize("name", ["beam", "llama13b", "tiny"])
def test_shared_pages_flag_changes_nothing(name):
    """PA_DECODE_SHARED_PAGES only changes the cache policy: same bits out."""
    x = wl.make_inputs(name, **SMALL[name])
    a, _ = gpu_step(x)
    b, _ = gpu_step(x, shared_pages=True)
    assert torch.equal(a, b)
    check_case(x)


@pytest.mark.parametrize("name,pt", [("llama7b", 0), ("llama7b", 256), ("gqa70b", 1024), ("beam", 0)])
def test_dispatch_order_changes_nothing(name, pt):
    """seq_order only reorders dispatch: every row is bitwise the same."""
    from paged_kv_cache_321_amd import binding
    x = wl.make_inputs(name, **SMALL[name])
    a, _ = gpu_step(x, partition_tokens=pt)
    order = binding.longest_first(x.plan.context_lens)
    b, _ = gpu_step(x, partition_tokens=pt, seq_order=order)
    assert torch.equal(a, b)
    rev = torch.arange(x.plan.num_seqs - 1, -1, -1, dtype=torch.int32, device="cuda")
    c, _ = gpu_step(x, partition_tokens=pt, seq_order=rev)
    assert torch.equal(a, c)


@pytest.mark.parametrize("n", [2, 64, 65, 200, 256, 257])
@pytest.mark.parametrize("hkv,group", [(4, 1), (2, 4)])
def test_in_kernel_longest_first(n, hkv, group):
    """Without seq_order a batch of at most 256 sequences (pages not shared)
    is dispatched longest context first, each workgroup ranking the lengths
    itself over up to four 64-lane windows (257 keeps the natural order):
    rows are the bits of the natural order and match the oracle.  Contexts
    0-600 with repeats (ties rank by index) and partitions of 64 tokens."""
    spec = wl.Spec(f"rank{n}x{group}", hkv * group, hkv, 128, 16, "bf16", seed=97)
    gen = torch.Generator().manual_seed(n)
    ctx = torch.randint(0, 601, (n,), generator=gen).tolist()
    ctx[n // 2] = ctx[0]
    x = wl.build_inputs(spec, wl.uniform_plan(ctx, 16, gen, new_tokens=True))
    a, _ = gpu_step(x, partition_tokens=64)
    ident = torch.arange(n, dtype=torch.int32, device="cuda")
    b, _ = gpu_step(x, partition_tokens=64, seq_order=ident)
    assert torch.equal(a, b)
    ref, _, _ = oracle_step(x)
    assert_close(as_f64(a), ref, "bf16", spec.name)


@pytest.mark.parametrize("name,pt", [("llama7b", 64), ("gqa70b", 1024)])
def test_workspace_reuse(name, pt):
    """One caller-owned workspace serves repeated multi-partition calls."""
    from paged_kv_cache_321_amd import binding
    x = wl.make_inputs(name, **SMALL[name])
    t = on_device(x)
    spec, plan = x.spec, x.plan
    code = binding.PA_BF16 if spec.dtype == "bf16" else binding.PA_F32
    n = binding.pa_decode_workspace_size(plan.num_seqs, spec.num_heads, spec.num_kv_heads,
                                         spec.head_dim, plan.block_size, plan.max_context_len,
                                         code, pt)
    assert n > 0
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")  # contents never matter
    if t["slot_mapping"].shape[0]:  # store the new tokens first (their slots hold NaN)
        binding.pa_reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"],
                                     t["slot_mapping"])
    outs = []
    for _ in range(3):
        out = torch.empty_like(t["q"])
        binding.pa_decode(out, t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                          t["context_lens"], x.scale, x.max_context_len, partition_tokens=pt,
                          workspace=ws)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref, _, _ = oracle_step(x)
    assert_close(as_f64(outs[0]), ref, spec.dtype, name)


def test_repeat_is_deterministic():
    x = wl.make_inputs("beam", **SMALL["beam"])
    a, _ = gpu_step(x)
    b, _ = gpu_step(x)
    assert torch.equal(a, b)


def test_poisoned_pool_gives_finite_output():
    x = wl.make_inputs("llama7b", **SMALL["llama7b"])
    assert torch.isnan(x.k_cache.float()).any()
    out, _ = gpu_step(x)
    assert torch.isfinite(out.float()).all()


def test_copy_on_write_leaves_source_unchanged():
    x = wl.make_inputs("beam", **SMALL["beam"])
    t = on_device(x)
    before_k = t["k_cache"].clone()
    out, t = gpu_step(x, t)
    pairs = x.plan.block_pairs
    assert len(pairs) > 0
    for src, dst in pairs:
        # Raw bits: the unused slots hold NaN, which never compares equal.
        assert np.array_equal(bits(t["k_cache"][src]), bits(before_k[src]))
    # Outside the copied-into and written blocks nothing changed.
    touched = set(pairs[:, 1].tolist()) | {int(s) // x.plan.block_size for s in x.plan.slot_mapping}
    rest = torch.tensor([b for b in range(x.plan.num_blocks) if b not in touched], device="cuda")
    assert np.array_equal(bits(t["k_cache"][rest]), bits(before_k[rest]))


# Block shapes whose 16-byte chunk count is below one slice (64), not a
# multiple of one (640 = 5 x 128), several slices (10240), and above the
# grid's 64 slices per pair (131072: the stride loop wraps).
@pytest.mark.parametrize("hkv,bs,d,dtype", [(1, 16, 64, torch.uint8), (5, 16, 64, torch.bfloat16),
                                             (40, 16, 128, torch.bfloat16), (128, 32, 128, torch.float32)])
def test_copy_blocks_bitwise_block_shapes(hkv, bs, d, dtype):
    import oracle.paged_attention as op
    g = torch.Generator().manual_seed(hkv * 1000 + bs + d)
    nb = 12
    shape = (nb, hkv, bs, d)
    if dtype == torch.uint8:
        k = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
        v = torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)
        kd, vd = k.view(torch.float8_e4m3fn).cuda(), v.view(torch.float8_e4m3fn).cuda()
    else:
        k = torch.randn(shape, generator=g).to(dtype)
        v = torch.randn(shape, generator=g).to(dtype)
        kd, vd = k.cuda(), v.cuda()
    ids = torch.randperm(nb, generator=g)
    pairs = torch.stack([ids[:5], ids[5:10]], 1).to(torch.int64)
    binding.pa_copy_blocks(kd, vd, pairs.cuda())
    torch.cuda.synchronize()
    kc, vc = wl.to_host_numpy(k).copy(), wl.to_host_numpy(v).copy()
    op.copy_blocks(kc, vc, pairs.numpy())
    assert np.array_equal(bits(kd), bits(kc))
    assert np.array_equal(bits(vd), bits(vc))


def test_bad_device_values_give_nan_rows_only():
    x = wl.make_inputs("llama7b", num_seqs=4, ctx_range=(40, 300))
    t = on_device(x)
    t["block_tables"][1, 0] = x.plan.num_blocks + 5          # out-of-range block id
    t["context_lens"][2] = x.max_context_len + 1             # longer than announced
    out, _ = gpu_step(x, t)
    o = out.float()
    assert torch.isnan(o[1]).all() and torch.isnan(o[2]).all()
    ref, _, _ = oracle_step(x)
    assert_close(as_f64(out)[[0, 3]], ref[[0, 3]], "bf16", "untouched rows")


def test_reshape_skips_negative_and_out_of_range_slots():
    x = wl.make_inputs("tiny")
    t = on_device(x)
    t["slot_mapping"][0] = -1
    t["slot_mapping"][2] = x.plan.num_blocks * x.plan.block_size  # one past the end
    before = t["k_cache"].clone()
    from paged_kv_cache_321_amd import binding
    binding.pa_reshape_and_cache(t["key"], t["value"], t["k_cache"], t["v_cache"], t["slot_mapping"])
    torch.cuda.synchronize()
    import oracle.paged_attention as op
    kc = x.k_cache.numpy().copy()
    vc = x.v_cache.numpy().copy()
    slots = x.plan.slot_mapping.copy()
    slots[0] = -1
    keep = np.array([0, 1, 3])  # slot 2 (out of range) is skipped by the kernel
    slots_k = slots[keep]
    op.reshape_and_cache(x.key.numpy()[keep], x.value.numpy()[keep], kc, vc, slots_k)
    assert np.array_equal(bits(t["k_cache"]), bits(kc))
    assert np.array_equal(bits(t["v_cache"]), bits(vc))
    assert np.array_equal(bits(before), bits(x.k_cache))


# ----------------------------------------------------------------------------
# Full-size workloads, sampled.
# ----------------------------------------------------------------------------

FULL = ["llama7b", "llama13b", "gqa70b", "beam"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    torch.cuda.empty_cache()
    x = wl.make_inputs(name, device="cuda", poison=True)
    s = x.plan.num_seqs
    g = torch.Generator().manual_seed(77)
    seqs = sorted(torch.randperm(s, generator=g)[:min(s, 4)].tolist())
    ref, ids, kc, vc = sampled_reference(x, seqs)
    # The inputs already live on the device: run the step in place on them.
    resident = {n: getattr(x, n) for n in ("q", "k_cache", "v_cache", "key", "value",
                                           "slot_mapping", "block_tables", "context_lens",
                                           "block_pairs")}
    out, t = gpu_step(x, t=resident)
    idx = torch.tensor(ids, device="cuda")
    assert np.array_equal(bits(t["k_cache"].index_select(0, idx)), bits(kc))
    assert np.array_equal(bits(t["v_cache"].index_select(0, idx)), bits(vc))
    assert_close(as_f64(out)[seqs], ref, x.spec.dtype, name)
    assert torch.isfinite(out.float()).all()
    del x, t, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("h,hkv,bs,kv", [(64, 8, 32, "bf16"), (64, 8, 32, "fp8"), (40, 40, 16, "bf16")])
def test_long_contexts_sampled(h, hkv, bs, kv):
    """Contexts of up to 128K tokens (4096-8192 pages per sequence, 32-64
    partitions, many page-id windows), ragged, on both decode paths and an
    E4M3 cache; the oracle checks every head of each sequence."""
    torch.cuda.empty_cache()
    spec = wl.Spec(f"long{h}x{hkv}x{bs}{kv}", h, hkv, 128, bs, "bf16", seed=h + bs,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    ctx = [131072, 65537] if hkv < h else [100001]
    plan = wl.uniform_plan(ctx, bs, torch.Generator().manual_seed(spec.seed), new_tokens=True)
    x = wl.build_inputs(spec, plan, device="cuda", poison=True)
    seqs = list(range(len(ctx)))
    ref, ids, kc, vc = sampled_reference(x, seqs)
    resident = {n: getattr(x, n) for n in ("q", "k_cache", "v_cache", "key", "value",
                                           "slot_mapping", "block_tables", "context_lens",
                                           "block_pairs")}
    out, t = gpu_step(x, t=resident)
    assert_close(as_f64(out), ref, x.spec.dtype, spec.name)
    del x, t, out
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# swap_blocks: device pool <-> pinned host pool.
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["llama7b", "gqa70b_fp8"])
def test_swap_out_and_in_bitwise(name):
    import oracle.paged_attention as op
    from paged_kv_cache_321_amd import binding
    from paged_kv_cache_321_amd.workloads import to_host_numpy
    x = wl.make_inputs(name, **SMALL[name])
    t = on_device(x)
    nb = x.plan.num_blocks
    host_k = torch.zeros((nb // 2 + 3,) + tuple(x.k_cache.shape[1:]), dtype=x.k_cache.dtype).pin_memory()
    host_v = torch.zeros_like(host_k).pin_memory()
    g = torch.Generator().manual_seed(9)
    src = torch.randperm(nb, generator=g)[:nb // 2]
    dst = torch.randperm(host_k.shape[0], generator=g)[:nb // 2]
    out_pairs = torch.stack([src, dst], 1).to(torch.int64)
    # Oracle on host copies taken before any GPU work.
    ok, ov = to_host_numpy(host_k).copy(), to_host_numpy(host_v).copy()
    op.swap_blocks(to_host_numpy(x.k_cache), to_host_numpy(x.v_cache), ok, ov, out_pairs.numpy())
    binding.pa_swap_blocks(host_k, host_v, t["k_cache"], t["v_cache"], out_pairs.to("cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(bits(host_k), bits(ok)) and np.array_equal(bits(host_v), bits(ov))
    # Back in, to other device blocks, with the pairs in pinned host memory and
    # one pair out of range (skipped).
    back = torch.randperm(nb, generator=g)[:nb // 2]
    in_pairs = torch.stack([dst, back], 1).to(torch.int64)
    in_pairs = torch.cat([in_pairs, torch.tensor([[0, nb + 3]])]).pin_memory()
    dk, dv = to_host_numpy(x.k_cache).copy(), to_host_numpy(x.v_cache).copy()  # swap-out only read it
    op.swap_blocks(ok, ov, dk, dv, in_pairs.numpy()[:-1])
    binding.pa_swap_blocks(t["k_cache"], t["v_cache"], host_k, host_v, in_pairs)
    torch.cuda.synchronize()
    assert np.array_equal(bits(t["k_cache"]), bits(dk)) and np.array_equal(bits(t["v_cache"]), bits(dv))


# ----------------------------------------------------------------------------
# Pools past 2^31 elements: every element offset into the caches needs 64 bits.
# ----------------------------------------------------------------------------

# (H, Hkv, BS, cache): pools of 2.29e9 elements per cache (4.6 GB bf16, 2.3 GB E4M3)
BIG_POOLS = [(40, 40, 16, "bf16"), (64, 8, 32, "bf16"), (64, 8, 32, "fp8")]


@pytest.mark.parametrize("h,hkv,bs,kv", BIG_POOLS)
def test_pool_past_2g_elements(h, hkv, bs, kv):
    torch.cuda.empty_cache()
    d = 128
    per_block = hkv * bs * d
    nb = (2_290_000_000 + per_block - 1) // per_block
    spec = wl.Spec(f"bigpool{h}x{hkv}x{bs}{kv}", h, hkv, d, bs, "bf16", seed=h + bs + 3,
                   kv_dtype=None if kv == "bf16" else kv, **wl.fp8_scales(kv))
    ctx = [1, 700, 2049, 5000]
    plan = wl.uniform_plan(ctx, bs, torch.Generator().manual_seed(spec.seed), new_tokens=True)
    plan = to_top_of_pool(plan, nb)
    used_min = int(plan.block_tables[plan.block_tables >= 0].min())
    assert used_min * per_block > 2 ** 31  # every page lies past 2^31 elements
    x = wl.build_inputs(spec, plan, device="cuda", poison=True)
    seqs = list(range(len(ctx)))
    ref, ids, kc, vc = sampled_reference(x, seqs)
    resident = {n: getattr(x, n) for n in ("q", "k_cache", "v_cache", "key", "value",
                                           "slot_mapping", "block_tables", "context_lens",
                                           "block_pairs")}
    out, t = gpu_step(x, t=resident)
    idx = torch.tensor(ids, device="cuda")
    assert np.array_equal(bits(t["k_cache"].index_select(0, idx)), bits(kc))
    assert np.array_equal(bits(t["v_cache"].index_select(0, idx)), bits(vc))
    assert_close(as_f64(out), ref, x.spec.dtype, spec.name)
    # copy_blocks from the top of the pool to a block just below 2^31 elements
    # and to the block just below the used ones.
    low = 2 ** 31 // per_block - 2
    src = [int(plan.block_tables[3, 0]), int(plan.block_tables[2, 1])]
    dst = [low, nb - 1 - len(ids) - 1]
    pairs = torch.tensor(list(zip(src, dst)), dtype=torch.int64, device="cuda")
    binding.pa_copy_blocks(t["k_cache"], t["v_cache"], pairs)
    torch.cuda.synchronize()
    for a, b in zip(src, dst):
        assert np.array_equal(bits(t["k_cache"][b]), bits(t["k_cache"][a]))
        assert np.array_equal(bits(t["v_cache"][b]), bits(t["v_cache"][a]))
    del x, t, out, resident
    torch.cuda.empty_cache()

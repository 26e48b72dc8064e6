"""GPU parity of the prefill kernel (bf16 caches with 4-bit K codes in groups
of 64, from 96 query rows per kv head: blocks of 128 rows sharing each
decoded tile) against the oracle, every output element:

- row counts at the threshold (96), one whole block (128), a ragged last
  block (200 rows: 128 + 72), many blocks (1200 rows over a cache that holds
  only the chunk itself, T = L); several batch entries and kv heads;
- causal and not, the ragged last tile, one split (outputs stored by the
  attention kernel), automatic and explicit splits (records merged by the
  merge kernel), with and without the rotation, the page's rotation
  precision;
- boolean masks with rows that keep no key, additive masks in fp32 and in
  the cache dtype;
- V values far beyond the fp16 range of the value operands (the per-group
  powers of two);
- the one-call step with a chunk of 16 appended rows (append kernel, then
  the prefill kernel): rows bit-exact, outputs within the tolerance;
- the other layouts it takes, with one and with several key splits (records
  of head_dim 64, 128 and 256): head_dim 64, 128 and 256 with 2-, 3- and 4-bit V
  codes (4-bit: the fp16 value operand and its residual), masks (rows that
  keep no key take the mean of their keys in the merge too), large V values,
  and a call whose 256 workgroups take the automatic
  plan.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O

pytestmark = pytest.mark.gpu

ATOL = 2e-3
rbq = pytest.importorskip("rotated_bit_quantized_amd")

NAMES = (("k_words", "kw"), ("k_scales", "ks"), ("k_biases", "kb"),
         ("v_words", "vw"), ("v_scales", "vs"), ("v_biases", "vb"))


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def _pair(dev, seed, B, Hkv, T, rot_mode="printed", rr=False, vscale=1.0):
    blocks = None
    rot = None
    if rot_mode is not None:
        blocks = O.rotation_blocks(W.rotation_draws(seed, 256), mode=rot_mode)
        if rr:
            blocks = O.round_to_dtype(blocks, "bf16")
        rot = rbq.build_block_so4(256, seed, dev, two_sided=rot_mode == "two_sided",
                                  round_to=torch.bfloat16 if rr else None)
        np.testing.assert_array_equal(rot.cpu().numpy(), blocks)
    g = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot, round_rotated=rr)
    o = O.QuantKVCache(k_bits=4, v_bits=3, dtype="bf16", group=64, round_rotated=rr)
    if T > 0:
        k = W.random_rows([seed, 1], (B, Hkv, T, 256), "bf16", "student_t3")
        v = W.random_rows([seed, 2], (B, Hkv, T, 256), "bf16", scale=vscale)
        g.append(k.to(dev), v.to(dev))
        o.append(k.float().numpy(), v.float().numpy(), blocks)
    return g, o, blocks


def _append_chunk(g, o, blocks, dev, seed, L, vscale=1.0):
    B, Hkv = g.desc.B, g.desc.H_kv
    kn = W.random_rows([seed, 3], (B, Hkv, L, 256), "bf16", "student_t3")
    vn = W.random_rows([seed, 4], (B, Hkv, L, 256), "bf16", scale=vscale)
    g.append(kn.to(dev), vn.to(dev))
    o.append(kn.float().numpy(), vn.float().numpy(), blocks)


# (B, H_q, H_kv, L, T0 cached before the chunk, causal, splits, rotation, rounded)
CASES = [
    (1, 16, 2, 12, 300, True, 0, "printed", False),     # 96 rows: the threshold
    (2, 16, 2, 16, 500, True, 0, "printed", False),     # 128 rows: one block
    (1, 8, 2, 50, 133, True, 3, "two_sided", False),    # 200 rows: 128 + 72
    (1, 4, 1, 300, 0, True, 1, "printed", True),        # 1200 rows, T = L
    (2, 16, 2, 64, 700, False, 0, "printed", False),    # not causal
    (1, 16, 2, 16, 2000, True, 5, None, False),         # no rotation, 5 splits
    (1, 16, 2, 24, 777, True, 1, "printed", True),      # one split, rounded rotation
]


def _cid(c):
    return "B{}_H{}-{}_L{}_T{}_{}_s{}_{}{}".format(
        c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full", c[6], c[7] or "norot",
        "_rr" if c[8] else "")


@pytest.mark.parametrize("case", CASES, ids=_cid)
def test_prefill_against_oracle(case, dev):
    B, Hq, Hkv, L, T0, causal, splits, rot_mode, rr = case
    print(f"[prefill] {_cid(case)}", flush=True)
    g, o, blocks = _pair(dev, 90, B, Hkv, T0, rot_mode, rr)
    _append_chunk(g, o, blocks, dev, 90, L)
    q = W.random_rows([91, L], (B, Hq, L, 256), "bf16")
    out = g.attend(q.to(dev), scale=1 / 16, causal=causal, splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    want = O.attention(q.float().numpy(), o, 1 / 16, causal, blocks)
    err = float(np.abs(got - want).max())
    assert err <= ATOL, err


@pytest.mark.parametrize("splits", [1, 0, 4])
@pytest.mark.parametrize("kind", ["bool", "f32", "dtype"])
def test_prefill_masks(kind, splits, dev):
    B, Hq, Hkv, L, T0 = 2, 16, 2, 16, 400
    print(f"[prefill mask] {kind} splits={splits}", flush=True)
    g, o, blocks = _pair(dev, 92, B, Hkv, T0)
    _append_chunk(g, o, blocks, dev, 92, L)
    T = T0 + L
    q = W.random_rows([93, 0], (B, Hq, L, 256), "bf16")
    rng = np.random.default_rng(94)
    if kind == "bool":
        m = rng.random((B, Hq, L, T)) < 0.4
        m[0, 3, 5, :] = False          # one row keeps no key
        m[1, :, 0, :] = False          # row 0 of every head of batch entry 1
        mask, ref_mask = torch.from_numpy(m), m
    else:
        m = rng.normal(0.0, 2.0, size=(B, Hq, L, T)).astype(np.float32)
        if kind == "dtype":
            mask = torch.from_numpy(m).to(torch.bfloat16)
            ref_mask = mask.float().numpy().astype(np.float64)
        else:
            mask, ref_mask = torch.from_numpy(m), m
    out = g.attend(q.to(dev), scale=1 / 16, causal=True, mask=mask.to(dev), splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    want = O.attention(q.float().numpy(), o, 1 / 16, True, blocks, mask=ref_mask)
    err = float(np.abs(got - want).max())
    assert err <= ATOL, err


@pytest.mark.parametrize("vscale", [1e5, 3e30])
def test_prefill_large_value_range(vscale, dev):
    print(f"[prefill large V] x{vscale:g}", flush=True)
    B, Hq, Hkv, L, T0 = 1, 16, 2, 16, 600
    g, o, blocks = _pair(dev, 95, B, Hkv, T0, vscale=vscale)
    _append_chunk(g, o, blocks, dev, 95, L, vscale=vscale)
    q = W.random_rows([96, 0], (B, Hq, L, 256), "bf16")
    for splits in (1, 0):
        out = g.attend(q.to(dev), scale=1 / 16, causal=True, splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        want = O.attention(q.float().numpy(), o, 1 / 16, True, blocks)
        err = float(np.abs(got - want).max()) / vscale
        assert err <= ATOL, (splits, err)


def test_prefill_one_call_step(dev):
    print("[prefill] one-call step, 16 appended rows", flush=True)
    B, Hq, Hkv, L, T0 = 2, 16, 2, 16, 321
    g, o, blocks = _pair(dev, 97, B, Hkv, T0)
    kn = W.random_rows([97, 3], (B, Hkv, L, 256), "bf16", "student_t3")
    vn = W.random_rows([97, 4], (B, Hkv, L, 256), "bf16")
    q = W.random_rows([97, 5], (B, Hq, L, 256), "bf16")
    out = g.append_attend(kn.to(dev), vn.to(dev), q.to(dev), scale=1 / 16, causal=True)
    torch.cuda.synchronize()
    o.append(kn.float().numpy(), vn.float().numpy(), blocks)
    rows = g.rows()
    for name, oname in NAMES:
        got = rows[name].cpu()
        got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
        bad = np.argwhere(got != o.arrays[oname][:, :, :o.offset])
        assert bad.size == 0, f"{name}: {len(bad)} mismatches"
    want = O.attention(q.float().numpy(), o, 1 / 16, True, blocks)
    err = float(np.abs(out.cpu().numpy() - want).max())
    assert err <= ATOL, err


def test_prefill_plan_is_used(dev):
    # the prefill kernel's plan: one split once the (b, kv head, 128-row
    # block) workgroups fill the compute units, key splits below that
    g, _, _ = _pair(dev, 98, 1, 2, 10240)
    assert rbq.rbq_quant_attn_splits(g.desc, 16, 2048) == 1
    assert rbq.rbq_quant_attn_splits(g.desc, 16, 16) > 1


# other layouts the prefill kernel takes (bf16, 4-bit K in groups of 64; groups
# of 128 and fp16 caches below): one
# key split (outputs stored by the attention kernel), explicit and automatic
# splits (records of head_dim 64, 128 or 256 merged by the merge kernel):
# (head_dim, v_bits, B, H_q, H_kv, L, T0, causal, splits, rotation, rounded)
LAYOUTS = [
    (128, 4, 1, 16, 2, 16, 300, True, 1, "two_sided", False),
    (128, 3, 1, 8, 2, 50, 133, True, 1, "printed", True),
    (128, 2, 2, 16, 2, 12, 200, False, 1, "printed", False),
    (256, 4, 1, 16, 2, 16, 250, True, 1, "two_sided", False),
    (256, 2, 1, 16, 2, 12, 180, True, 1, None, False),
    (128, 4, 2, 16, 8, 1024, 76, True, 0, "two_sided", False),  # 256 workgroups: automatic plan
    (128, 4, 1, 16, 2, 16, 3000, True, 0, "two_sided", False),  # automatic splits, records
    (128, 3, 2, 8, 2, 50, 700, True, 5, "printed", True),
    (128, 2, 1, 16, 2, 40, 2600, False, 0, "printed", False),
    (256, 4, 1, 16, 2, 16, 2500, True, 0, "two_sided", False),
    (256, 2, 1, 16, 2, 12, 1800, True, 7, None, False),
    (64, 4, 1, 16, 2, 16, 300, True, 1, "two_sided", False),    # head_dim 64: one group
    (64, 3, 2, 8, 2, 50, 700, True, 0, "printed", True),
    (64, 2, 1, 16, 2, 40, 1000, False, 3, None, False),
    # head_dim 64 with an odd key count: the last key's 2-byte scales share a
    # word with the key past the end
    (64, 2, 2, 8, 1, 15, 338, True, 0, "two_sided", True),
    (64, 4, 1, 16, 2, 12, 301, False, 1, None, False),
]


def _lid(c):
    return "D{}_v{}_B{}_H{}-{}_L{}_T{}_{}_s{}_{}{}".format(
        c[0], c[1], c[2], c[3], c[4], c[5], c[6], "causal" if c[7] else "full", c[8], c[9] or "norot",
        "_rr" if c[10] else "")


def _layout_pair(dev, seed, D, vb, B, Hkv, T, rot_mode, rr, vscale=1.0, dtype="bf16", group=64):
    tdt = W._TORCH_DTYPES[dtype]
    blocks = rot = None
    if rot_mode is not None:
        blocks = O.rotation_blocks(W.rotation_draws(seed, D), mode=rot_mode)
        if rr:
            blocks = O.round_to_dtype(blocks, dtype)
        rot = rbq.build_block_so4(D, seed, dev, two_sided=rot_mode == "two_sided",
                                  round_to=tdt if rr else None)
    g = rbq.RotatedQuantKVCache(B, Hkv, dtype=tdt, device=dev, rot=rot, head_dim=D, group_size=group,
                                k_bits=4, v_bits=vb, round_rotated=rr)
    o = O.QuantKVCache(k_bits=4, v_bits=vb, dtype=dtype, group=group, round_rotated=rr)
    k = W.random_rows([seed, 1], (B, Hkv, T, D), dtype, "student_t3")
    v = W.random_rows([seed, 2], (B, Hkv, T, D), dtype, scale=vscale)
    g.append(k.to(dev), v.to(dev))
    o.append(k.float().numpy(), v.float().numpy(), blocks)
    return g, o, blocks


@pytest.mark.parametrize("case", LAYOUTS, ids=_lid)
def test_prefill_other_layouts(case, dev):
    D, vb, B, Hq, Hkv, L, T0, causal, splits, rot_mode, rr = case
    print(f"[prefill layout] {_lid(case)}", flush=True)
    g, o, blocks = _layout_pair(dev, 70, D, vb, B, Hkv, T0 + L, rot_mode, rr)
    q = W.random_rows([71, L], (B, Hq, L, D), "bf16")
    out = g.attend(q.to(dev), scale=D ** -0.5, causal=causal, splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    want = O.attention(q.float().numpy(), o, D ** -0.5, causal, blocks)
    err = float(np.abs(got - want).max())
    assert err <= ATOL, err


@pytest.mark.parametrize("splits", [1, 0])
@pytest.mark.parametrize("kind", ["bool", "f32"])
def test_prefill_other_layout_masks(kind, splits, dev):
    D, vb, B, Hq, Hkv, L, T = 128, 4, 2, 16, 2, 16, 2333
    print(f"[prefill layout mask] {kind} splits={splits}", flush=True)
    g, o, blocks = _layout_pair(dev, 72, D, vb, B, Hkv, T, "two_sided", False)
    q = W.random_rows([73, 0], (B, Hq, L, D), "bf16")
    rng = np.random.default_rng(74)
    if kind == "bool":
        m = rng.random((B, Hq, L, T)) < 0.4
        m[0, 3, 5, :] = False
        m[1, :, 0, :] = False
    else:
        m = rng.normal(0.0, 2.0, size=(B, Hq, L, T)).astype(np.float32)
    out = g.attend(q.to(dev), scale=D ** -0.5, causal=True, mask=torch.from_numpy(m).to(dev),
                   splits=splits)
    torch.cuda.synchronize()
    if splits == 0:
        assert rbq.rbq_quant_attn_splits(g.desc, Hq, L) > 1
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    want = O.attention(q.float().numpy(), o, D ** -0.5, True, blocks, mask=m)
    err = float(np.abs(got - want).max())
    assert err <= ATOL, err


def test_prefill_other_layout_large_values(dev):
    # 4-bit V codes: V' and its residual carry code x scale exactly
    print("[prefill layout] large V", flush=True)
    D, vb, B, Hq, Hkv, L, T = 128, 4, 1, 16, 2, 16, 400
    g, o, blocks = _layout_pair(dev, 75, D, vb, B, Hkv, T, "printed", False, vscale=1e5)
    q = W.random_rows([76, 0], (B, Hq, L, D), "bf16")
    want = O.attention(q.float().numpy(), o, D ** -0.5, True, blocks)
    for splits in (1, 3):
        out = g.attend(q.to(dev), scale=D ** -0.5, causal=True, splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        err = float(np.abs(got - want).max()) / 1e5
        assert err <= ATOL, (splits, err)


# fp16 caches (the scales and biases in fp16: V' and its exact residual for
# every V width, the K biases as bf16 hi and lo parts in the bias product):
# (head_dim, v_bits, B, H_q, H_kv, L, T0, causal, splits, rotation, rounded)
FP16_CASES = [
    (256, 3, 1, 16, 2, 16, 300, True, 1, "printed", False),   # the default layout
    (256, 3, 2, 8, 2, 50, 700, True, 0, "two_sided", True),
    (128, 4, 1, 16, 2, 16, 3000, True, 0, "two_sided", False),
    (128, 2, 1, 16, 2, 12, 200, False, 3, "printed", False),
    (64, 2, 1, 16, 2, 15, 338, True, 0, None, False),          # odd key count
    (64, 3, 2, 8, 1, 20, 400, True, 1, "printed", True),
]


@pytest.mark.parametrize("case", FP16_CASES, ids=_lid)
def test_prefill_fp16_caches(case, dev):
    D, vb, B, Hq, Hkv, L, T0, causal, splits, rot_mode, rr = case
    print(f"[prefill fp16] {_lid(case)}", flush=True)
    g, o, blocks = _layout_pair(dev, 80, D, vb, B, Hkv, T0 + L, rot_mode, rr, dtype="f16")
    q = W.random_rows([81, L], (B, Hq, L, D), "f16")
    out = g.attend(q.to(dev), scale=D ** -0.5, causal=causal, splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    want = O.attention(q.float().numpy(), o, D ** -0.5, causal, blocks)
    err = float(np.abs(got - want).max())
    assert err <= ATOL, err


@pytest.mark.parametrize("kind", ["bool", "f32", "f16"])
def test_prefill_fp16_masks(kind, dev):
    D, vb, B, Hq, Hkv, L, T = 256, 3, 2, 16, 2, 16, 1333
    print(f"[prefill fp16 mask] {kind}", flush=True)
    g, o, blocks = _layout_pair(dev, 82, D, vb, B, Hkv, T, "printed", False, dtype="f16")
    q = W.random_rows([83, 0], (B, Hq, L, D), "f16")
    rng = np.random.default_rng(84)
    if kind == "bool":
        m = rng.random((B, Hq, L, T)) < 0.4
        m[0, 3, 5, :] = False
        m[1, :, 0, :] = False
        md = torch.from_numpy(m)
    else:
        m = rng.normal(0.0, 2.0, size=(B, Hq, L, T)).astype(np.float32)
        md = torch.from_numpy(m)
        if kind == "f16":
            md = md.to(torch.float16)
            m = md.float().numpy()
    for splits in (1, 0):
        out = g.attend(q.to(dev), scale=D ** -0.5, causal=True, mask=md.to(dev), splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        want = O.attention(q.float().numpy(), o, D ** -0.5, True, blocks, mask=m)
        err = float(np.abs(got - want).max())
        assert err <= ATOL, (splits, err)


def test_prefill_fp16_large_values(dev):
    # fp16 V values near the top of the fp16 range: scales and biases times
    # the powers of two stay finite, the residual keeps code x scale exact
    print("[prefill fp16] large V", flush=True)
    D, vb, B, Hq, Hkv, L, T = 256, 3, 1, 16, 2, 16, 500
    g, o, blocks = _layout_pair(dev, 85, D, vb, B, Hkv, T, "printed", False, vscale=1e4, dtype="f16")
    q = W.random_rows([86, 0], (B, Hq, L, D), "f16")
    want = O.attention(q.float().numpy(), o, D ** -0.5, True, blocks)
    for splits in (1, 3):
        out = g.attend(q.to(dev), scale=D ** -0.5, causal=True, splits=splits)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        err = float(np.abs(got - want).max()) / 1e4
        assert err <= ATOL, (splits, err)


# groups of 128 dims (two 64-dim blocks of the kernel sharing a scale and a
# bias): (head_dim, v_bits, dtype, B, H_q, H_kv, L, T0, causal, splits, rotation, rounded)
G128_CASES = [
    (256, 3, "bf16", 1, 16, 2, 16, 300, True, 1, "printed", False),
    (256, 4, "bf16", 2, 8, 2, 50, 700, True, 0, "two_sided", True),
    (128, 2, "bf16", 1, 16, 2, 15, 338, True, 0, "two_sided", False),   # odd key count, 2-byte scales
    (128, 3, "f16", 1, 16, 2, 12, 201, False, 3, None, False),
    (256, 2, "f16", 1, 16, 2, 16, 1001, True, 0, "printed", False),
]


def _gid(c):
    return "D{}_v{}_{}_B{}_H{}-{}_L{}_T{}_{}_s{}_{}{}".format(
        c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], "causal" if c[8] else "full", c[9],
        c[10] or "norot", "_rr" if c[11] else "")


@pytest.mark.parametrize("case", G128_CASES, ids=_gid)
def test_prefill_groups_of_128(case, dev):
    D, vb, dtype, B, Hq, Hkv, L, T0, causal, splits, rot_mode, rr = case
    print(f"[prefill group 128] {_gid(case)}", flush=True)
    g, o, blocks = _layout_pair(dev, 90, D, vb, B, Hkv, T0 + L, rot_mode, rr, dtype=dtype, group=128)
    q = W.random_rows([91, L], (B, Hq, L, D), dtype)
    out = g.attend(q.to(dev), scale=D ** -0.5, causal=causal, splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    want = O.attention(q.float().numpy(), o, D ** -0.5, causal, blocks)
    err = float(np.abs(got - want).max())
    assert err <= ATOL, err


def test_prefill_groups_of_128_bool_mask(dev):
    D, vb, B, Hq, Hkv, L, T = 128, 4, 2, 16, 2, 16, 1333
    print("[prefill group 128] boolean mask", flush=True)
    g, o, blocks = _layout_pair(dev, 92, D, vb, B, Hkv, T, "two_sided", False, group=128)
    q = W.random_rows([93, 0], (B, Hq, L, D), "bf16")
    rng = np.random.default_rng(94)
    m = rng.random((B, Hq, L, T)) < 0.4
    m[0, 3, 5, :] = False
    m[1, :, 0, :] = False
    for splits in (1, 0):
        out = g.attend(q.to(dev), scale=D ** -0.5, causal=True, mask=torch.from_numpy(m).to(dev),
                       splits=splits)
        torch.cuda.synchronize()
        want = O.attention(q.float().numpy(), o, D ** -0.5, True, blocks, mask=m)
        err = float(np.abs(out.cpu().numpy() - want).max())
        assert err <= ATOL, (splits, err)

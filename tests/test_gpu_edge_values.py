"""GPU parity at the edges of the value range and of the mask, through the C
ABI, against the oracle:

- boolean masks that drop every key of some query rows: the SDPA on the
  quant_kv.py page fills dropped scores with the dtype's most negative value,
  so such a row weights all of its keys alike (the oracle's finfo.min fill);
  both attention kernels, one split (the output stored by the attention
  kernel) and several (stored by the merge kernel), with and without the
  causal mask;
- V values far beyond the fp16 range of the dedicated kernel's value
  operands (bf16 V ~ N(0,1) x 1e5, fp16 V ~ N(0,1) x 1e4): the outputs scale
  with V, so the tolerance is 2e-3 times the factor V was scaled by;
- groups whose range is about 1e-38 (bf16 scales in the fp32 subnormal
  range, where the reciprocal of the scale overflows): the rows written by
  the append kernel and by the attention kernel of the one-call step equal
  the oracle's bit for bit.
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


def _pair(dev, seed, B, Hkv, T, D=256, gs=64, kb=4, vb=3, dtype="bf16", kscale=1.0,
          vscale=1.0):
    tdt = W._TORCH_DTYPES[dtype]
    blocks = O.rotation_blocks(W.rotation_draws(seed, D))
    rot = rbq.build_block_so4(D, seed, dev)
    np.testing.assert_array_equal(rot.cpu().numpy(), blocks)
    g = rbq.RotatedQuantKVCache(B, Hkv, dtype=tdt, device=dev, rot=rot, head_dim=D,
                                group_size=gs, k_bits=kb, v_bits=vb)
    o = O.QuantKVCache(k_bits=kb, v_bits=vb, dtype=dtype, group=gs)
    k = W.random_rows([seed, 1], (B, Hkv, T, D), dtype, scale=kscale)
    v = W.random_rows([seed, 2], (B, Hkv, T, D), dtype, scale=vscale)
    g.append(k.to(dev), v.to(dev))
    o.append(k.float().numpy(), v.float().numpy(), blocks)
    return g, o, blocks


def _rows_equal(g, o, what):
    torch.cuda.synchronize()
    assert g.offset == o.offset
    rows = g.rows()
    for name, oname in NAMES:
        got = rows[name].cpu()
        got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
        bad = np.argwhere(got != o.arrays[oname][:, :, :o.offset])
        assert bad.size == 0, f"{what} {name}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


# (head_dim, group, k_bits, v_bits, dtype, B, H_q, H_kv, T, L): the dedicated
# kernel (8-row blocks) and the tile kernel in both shapes (one wave for up to
# 16 rows per kv head at head_dim 128 and up to 8 at head_dim 256 with 4
# groups, four waves otherwise)
MASK_CASES = [
    (256, 64, 4, 3, "bf16", 2, 16, 2, 1000, 4),
    (256, 64, 4, 3, "f16", 1, 8, 1, 333, 2),
    (128, 64, 4, 4, "bf16", 2, 8, 2, 700, 2),
    (128, 32, 5, 3, "f16", 1, 16, 2, 500, 4),
    (256, 64, 4, 4, "bf16", 1, 16, 2, 600, 3),
]


def _mid(c):
    return "D{}_g{}_k{}v{}_{}_B{}_H{}-{}_T{}_L{}".format(*c)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 0, 5])
@pytest.mark.parametrize("case", MASK_CASES, ids=_mid)
def test_all_masked_rows_average_every_key(case, splits, causal, dev):
    D, gs, kb, vb, dtype, B, Hq, Hkv, T, L = case
    print(f"[all-masked rows] {_mid(case)} splits={splits} causal={causal}", flush=True)
    g, o, blocks = _pair(dev, 81, B, Hkv, T, D, gs, kb, vb, dtype)
    q = W.random_rows([81, 3], (B, Hq, L, D), dtype)
    rng = np.random.default_rng(82)
    m = rng.random((B, Hq, L, T)) < 0.5
    m[..., 0] = True
    m[0, 1, L - 1, :] = False          # one row of one head
    m[B - 1, :, 0, :] = False          # row 0 of every head of the last batch entry
    m[0, Hq - 1, :, T // 2:] = False   # keys kept in the first half only
    out = g.attend(q.to(dev), scale=D ** -0.5, causal=causal,
                   mask=torch.from_numpy(m).to(dev), splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    want = O.attention(q.float().numpy(), o, D ** -0.5, causal, blocks, mask=m)
    err = float(np.abs(got - want).max())
    assert err <= ATOL, err


@pytest.mark.parametrize("dtype,vscale", [("bf16", 1e5), ("bf16", 3e30), ("f16", 1e4)])
@pytest.mark.parametrize("splits", [1, 0])
def test_large_value_range(dtype, vscale, splits, dev):
    # scales and biases far above the fp16 range of the value operands (and,
    # for fp16 caches, codes times scales above 65504)
    print(f"[large V] {dtype} x{vscale:g} splits={splits}", flush=True)
    B, Hq, Hkv, T = 2, 16, 2, 1500
    g, o, blocks = _pair(dev, 83, B, Hkv, T, dtype=dtype, vscale=vscale)
    q = W.random_rows([83, 3], (B, Hq, 2, 256), dtype)
    out = g.attend(q.to(dev), scale=1 / 16, causal=True, splits=splits)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    want = O.attention(q.float().numpy(), o, 1 / 16, True, blocks)
    err = float(np.abs(got - want).max()) / vscale
    assert err <= ATOL, err


def test_large_values_in_the_one_call_step(dev):
    print("[large V] one-call step", flush=True)
    B, Hq, Hkv, T = 2, 16, 2, 900
    g, o, blocks = _pair(dev, 84, B, Hkv, T, vscale=1e5)
    kn = W.random_rows([84, 5], (B, Hkv, 1, 256), "bf16")
    vn = W.random_rows([84, 6], (B, Hkv, 1, 256), "bf16", scale=1e6)
    q = W.random_rows([84, 3], (B, Hq, 1, 256), "bf16")
    out = g.append_attend(kn.to(dev), vn.to(dev), q.to(dev), scale=1 / 16, causal=True)
    o.append(kn.float().numpy(), vn.float().numpy(), blocks)
    _rows_equal(g, o, "one-call step")
    want = O.attention(q.float().numpy(), o, 1 / 16, True, blocks)
    err = float(np.abs(out.cpu().numpy() - want).max()) / 1e6
    assert err <= ATOL, err


@pytest.mark.parametrize("n", [1, 8])
def test_tiny_groups_bit_exact(n, dev):
    # values about 1e-38: scales (range / 15 or / 7) in the fp32 subnormal
    # range, where x * rcp(s) is not finite and the exact division decides
    print(f"[tiny groups] n={n}", flush=True)
    B, Hq, Hkv, T = 1, 8, 2, 300
    g, o, blocks = _pair(dev, 85, B, Hkv, T, kscale=1e-38, vscale=3e-38)
    _rows_equal(g, o, "append kernel")
    kn = W.random_rows([85, 5], (B, Hkv, n, 256), "bf16", scale=2e-38)
    vn = W.random_rows([85, 6], (B, Hkv, n, 256), "bf16", scale=1e-38)
    q = W.random_rows([85, 3], (B, Hq, 1, 256), "bf16")
    out = g.append_attend(kn.to(dev), vn.to(dev), q.to(dev), scale=1 / 16, causal=True)
    o.append(kn.float().numpy(), vn.float().numpy(), blocks)
    _rows_equal(g, o, "one-call step")
    want = O.attention(q.float().numpy(), o, 1 / 16, True, blocks)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    assert float(np.abs(got - want).max()) <= ATOL


def test_all_masked_rows_with_128_splits(dev):
    # a long key range over few (b, kv head) units: 128 key splits merged by
    # the merge kernel's 4 thread groups in two rounds, rows that keep no key
    print("[all-masked rows] 128 splits", flush=True)
    B, Hq, Hkv, T, L = 1, 16, 2, 4096, 2
    g, o, blocks = _pair(dev, 85, B, Hkv, T)
    q = W.random_rows([85, 3], (B, Hq, L, 256), "bf16")
    rng = np.random.default_rng(86)
    m = rng.random((B, Hq, L, T)) < 0.5
    m[0, 2, 1, :] = False
    m[0, 9, 0, :] = False
    for mask, ref in ((torch.from_numpy(m), m), (None, None)):
        out = g.attend(q.to(dev), scale=1 / 16, causal=True, splits=128,
                       mask=None if mask is None else mask.to(dev))
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.isfinite(got).all()
        want = O.attention(q.float().numpy(), o, 1 / 16, True, blocks, mask=ref)
        err = float(np.abs(got - want).max())
        assert err <= ATOL, err

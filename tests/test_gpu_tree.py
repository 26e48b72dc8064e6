"""GPU: batched verification of draft paths (mtp/kv_cache.py ``tile_caches`` /
``commit_tree_row``) and the SDPA's array masks (quant_kv.py
``asym_quantized_sdpa``: boolean keep-masks and additive masks), against the
oracle: attention within 2e-3 max abs, cache arrays bit for bit."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O
import _ref as R

pytestmark = pytest.mark.gpu
ATOL = 2e-3

rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402

dev = torch.device("cuda:0")


@pytest.fixture(scope="module")
def blocks():
    return O.rotation_blocks(W.rotation_draws(W.ROTATION_SEED, 256))


@pytest.fixture(scope="module")
def rot():
    return rbq.build_block_so4(256, W.ROTATION_SEED, dev)


def _pair(seed, B, Hkv, T, blocks, rot, dtype="bf16"):
    k = W.random_rows([seed, 1], (B, Hkv, T, 256), dtype)
    v = W.random_rows([seed, 2], (B, Hkv, T, 256), dtype)
    g = rbq.RotatedQuantKVCache(B, Hkv, dtype=k.dtype, device=dev, rot=rot)
    g.append(k.to(dev), v.to(dev))
    o = O.QuantKVCache(dtype=dtype)
    o.append(k.float().numpy(), v.float().numpy(), blocks)
    return g, o


def _check(got, want, what):
    err = float(np.nanmax(np.abs(got.cpu().numpy() - want)))
    assert np.isfinite(got.cpu().numpy()).all(), what
    assert err <= ATOL, f"{what}: max abs error {err}"


@pytest.mark.parametrize("kind", ["bool_bcast_heads", "bool_2d", "add_f32_per_head",
                                  "add_dtype", "bool_with_causal"])
def test_masked_attention_matches_oracle(kind, blocks, rot):
    print(f"masked attention {kind}", flush=True)
    B, Hkv, Hq, T, L = 2, 2, 16, 1000, 4
    g, o = _pair(71, B, Hkv, T, blocks, rot)
    q = W.random_rows([71, 3], (B, Hq, L, 256), "bf16")
    rng = np.random.default_rng(72)
    causal = False
    if kind == "bool_bcast_heads":
        m = rng.random((B, 1, L, T)) < 0.6
        m[..., 5] = True
    elif kind == "bool_2d":
        m = rng.random((L, T)) < 0.3
        m[:, 999] = True
    elif kind == "add_f32_per_head":
        m = rng.normal(0, 2, (B, Hq, L, T)).astype(np.float32)
        m[rng.random((B, Hq, L, T)) < 0.2] = -np.inf
        m[..., 0] = 0.0
    elif kind == "add_dtype":
        m = torch.tensor(rng.normal(0, 1.5, (B, 1, L, T)), dtype=torch.float64).to(
            torch.bfloat16).float().numpy()
    else:
        m = rng.random((B, Hq, L, T)) < 0.5
        m[..., 0] = True
        causal = True
    mt = torch.from_numpy(m)
    if kind == "add_dtype":
        mt = mt.to(torch.bfloat16)
    out = g.attend(q.to(dev), causal=causal, mask=mt.to(dev))
    want = O.attention(q.float().numpy(), o, 1 / 16, causal, blocks, mask=m)
    _check(out, want, kind)


def test_causal_pattern_mask_equals_causal(blocks, rot):
    B, Hkv, Hq, T, L = 1, 2, 16, 777, 5
    g, _ = _pair(73, B, Hkv, T, blocks, rot)
    q = W.random_rows([73, 3], (B, Hq, L, 256), "bf16").to(dev)
    keep = torch.arange(T - L, T)[:, None] >= torch.arange(T)[None]
    a = g.attend(q, causal=True)
    b = g.attend(q, causal=False, mask=keep.to(dev))
    c = g.attend(q, causal=False, mask=torch.where(keep, 0.0, float("-inf")).float().to(dev))
    torch.cuda.synchronize()
    assert torch.allclose(a, b, atol=1e-6, rtol=0) and torch.allclose(a, c, atol=1e-6, rtol=0)


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_masked_split_independence(splits, blocks, rot):
    B, Hkv, Hq, T, L = 1, 2, 8, 2000, 2
    g, o = _pair(74, B, Hkv, T, blocks, rot)
    q = W.random_rows([74, 3], (B, Hq, L, 256), "bf16")
    m = np.random.default_rng(75).random((L, T)) < 0.5
    m[:, 3] = True
    out = g.attend(q.to(dev), causal=False, mask=torch.from_numpy(m).to(dev), splits=splits)
    want = O.attention(q.float().numpy(), o, 1 / 16, False, blocks, mask=m)
    _check(out, want, f"splits={splits}")


def test_fp16_cache_with_mask(blocks, rot):
    g, o = _pair(76, 1, 1, 256, blocks, rot, dtype="f16")
    q = W.random_rows([76, 3], (1, 1, 1, 256), "f16")
    m = np.random.default_rng(77).normal(0, 1, (1, 256)).astype(np.float16)
    out = g.attend(q.to(dev), mask=torch.from_numpy(m).to(dev))
    want = O.attention(q.float().numpy(), o, 1 / 16, True, blocks, mask=m.astype(np.float32))
    _check(out, want, "fp16 additive")


def test_tree_verification_flow(blocks, rot):
    """tile a batch-1 cache over P paths, append each path's draft tokens,
    verify all paths in one masked call (the draft tokens of a path form a
    small tree: token 2 and 3 both follow token 1), commit the winning path's
    accepted prefix; compare with the oracle run through the same steps."""
    print("tree verification flow", flush=True)
    P, Hkv, Hq, T0, L = 3, 2, 16, 300, 4
    g, o = _pair(78, 1, Hkv, T0, blocks, rot)
    rbq.tile_caches([g], P)
    O.tile_cache(o, P)
    assert g.desc.B == P and g.offset == T0
    torch.cuda.synchronize()
    for b in range(P):
        ref = {n: o.arrays[n][b, h, :T0] for n in ("kw", "ks", "kb", "vw", "vs", "vb") for h in [0]}
        for h in range(Hkv):
            refh = {n: o.arrays[n][b, h, :T0] for n in ("kw", "ks", "kb", "vw", "vs", "vb")}
            R.assert_slab_equal(R.device_rows(g, b, h), refh, f"tiled b={b} h={h}")
    kd = W.random_rows([79, 1], (P, Hkv, L, 256), "bf16")
    vd = W.random_rows([79, 2], (P, Hkv, L, 256), "bf16")
    g.append(kd.to(dev), vd.to(dev))
    o.append(kd.float().numpy(), vd.float().numpy(), blocks)
    T = T0 + L
    parent = [-1, 0, 1, 1]  # draft token i follows parent[i]
    keep = np.zeros((L, T), bool)
    keep[:, :T0] = True
    for i in range(L):
        j = i
        while j >= 0:
            keep[i, T0 + j] = True
            j = parent[j]
    q = W.random_rows([79, 3], (P, Hq, L, 256), "bf16")
    out = g.attend(q.to(dev), causal=False, mask=torch.from_numpy(keep).to(dev))
    want = O.attention(q.float().numpy(), o, 1 / 16, False, blocks, mask=keep)
    _check(out, want, "tree verify")
    assert rbq.commit_tree_row([g], L, 2, 1) is True
    assert O.commit_tree_row([o], L, 2, 1) is True
    torch.cuda.synchronize()
    assert g.desc.B == 1 and g.offset == o.offset == T0 + 2
    for h in range(Hkv):
        refh = {n: o.arrays[n][0, h, :o.offset] for n in ("kw", "ks", "kb", "vw", "vs", "vb")}
        R.assert_slab_equal(R.device_rows(g, 0, h), refh, f"committed h={h}")
    # decoding continues from the winning path
    k1 = W.random_rows([80, 1], (1, Hkv, 1, 256), "bf16")
    v1 = W.random_rows([80, 2], (1, Hkv, 1, 256), "bf16")
    g.append(k1.to(dev), v1.to(dev))
    o.append(k1.float().numpy(), v1.float().numpy(), blocks)
    q1 = W.random_rows([80, 3], (1, Hq, 1, 256), "bf16")
    _check(g.attend(q1.to(dev)), O.attention(q1.float().numpy(), o, 1 / 16, True, blocks),
           "decode after commit")
    with pytest.raises(ValueError):
        rbq.commit_tree_row([g], 1, 2, 0)
    with pytest.raises(ValueError):
        g.commit_row(1, 1, 5)
    g.tile(2)
    with pytest.raises(ValueError):
        g.tile(2)


def test_mask_argument_errors(rot):
    g = rbq.RotatedQuantKVCache(1, 2, device=dev, rot=rot)
    g.append(torch.zeros(1, 2, 10, 256, dtype=torch.bfloat16, device=dev),
             torch.zeros(1, 2, 10, 256, dtype=torch.bfloat16, device=dev))
    q = torch.zeros(1, 4, 1, 256, dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        g.attend(q, mask=torch.ones(1, 9, dtype=torch.bool, device=dev))  # too few keys
    with pytest.raises(ValueError):
        g.attend(q, mask=torch.ones(1, 10, dtype=torch.float64, device=dev))
    with pytest.raises(ValueError):
        g.attend(q, mask=torch.ones(1, 20, dtype=torch.bool, device=dev)[:, ::2])  # strided keys
    lib = capi.library()
    import ctypes
    out = torch.empty(1, 4, 1, 256, device=dev)
    m = torch.ones(1, 10, dtype=torch.bool, device=dev)
    st = lib.rbq_quant_attn_decode_mask(ctypes.byref(g.desc), q.data_ptr(), 4, 1, 0.0625, 1,
                                        m.data_ptr(), 9, 0, 0, 0, None, out.data_ptr(), 0, None,
                                        0, None)
    assert st == capi.RBQ_EINVAL
    st = lib.rbq_quant_attn_decode_mask(ctypes.byref(g.desc), q.data_ptr(), 4, 1, 0.0625, 1,
                                        m.data_ptr(), capi.RBQ_MASK_BOOL, -1, 0, 0, None,
                                        out.data_ptr(), 0, None, 0, None)
    assert st == capi.RBQ_EINVAL
    st = lib.rbq_quant_attn_decode_mask(ctypes.byref(g.desc), q.data_ptr(), 4, 1, 0.0625, 1,
                                        None, capi.RBQ_MASK_BOOL, 0, 0, 0, None,
                                        out.data_ptr(), 0, None, 0, None)
    assert st == capi.RBQ_EINVAL

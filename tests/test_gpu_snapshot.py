"""GPU: cache snapshots and their restore (the snapshot interface of the
quant_kv.py page and ``_snapshot`` / ``_restore`` / ``commit_verified_snapshot``
of mtp/kv_cache.py) through the C ABI's prefix copy, against the oracle's
cache run through the same sequence: rows [0, offset) of the six arrays bit
for bit, and the offset.  The copy itself is checked bit for bit on odd
capacities (4-byte path) and at the batched-decode size."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O
import _ref as R

pytestmark = pytest.mark.gpu

rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402

dev = torch.device("cuda:0")


@pytest.fixture(scope="module")
def blocks():
    return O.rotation_blocks(W.rotation_draws(W.ROTATION_SEED, 256))


@pytest.fixture(scope="module")
def rot():
    return rbq.build_block_so4(256, W.ROTATION_SEED, dev)


def _tokens(seed, B, H, n):
    return (W.random_rows([seed, 1], (B, H, n, 256), "bf16"),
            W.random_rows([seed, 2], (B, H, n, 256), "bf16"))


def _append(g, o, k, v, blocks):
    g.append(k.contiguous().to(dev), v.contiguous().to(dev))
    o.append(k.float().numpy(), v.float().numpy(), blocks)


def _assert_same(g, o, what):
    torch.cuda.synchronize()
    assert g.offset == o.offset, what
    if o.offset == 0:
        return
    B, H = g.desc.B, g.desc.H_kv
    for b in range(B):
        for h in range(H):
            ref = {n: o.arrays[n][b, h, :o.offset] for n in ("kw", "ks", "kb", "vw", "vs", "vb")}
            R.assert_slab_equal(R.device_rows(g, b, h), ref, f"{what} b={b} h={h}")


def test_restore_sequence_matches_oracle(rot, blocks):
    print("snapshot sequence B=2 H=2 T=300", flush=True)
    k, v = _tokens(41, 2, 2, 310)
    kx, vx = _tokens(42, 2, 2, 6)
    g = rbq.RotatedQuantKVCache(2, 2, device=dev, rot=rot)
    o = O.QuantKVCache()
    _append(g, o, k[:, :, :300], v[:, :, :300], blocks)
    gs, os_ = rbq.snapshot_caches([g]), O.snapshot([o])
    assert gs[0].offset == 300 and gs[0].meta_state == ("64", "4", "3")
    _append(g, o, k[:, :, 300:], v[:, :, 300:], blocks)
    assert g.trim(20) == o.trim(20) == 20
    _append(g, o, kx, vx, blocks)  # rewrites rows 290-295 that the snapshot covers
    _assert_same(g, o, "before restore")
    rbq.restore_caches([g], gs)
    O.restore([o], os_)
    _assert_same(g, o, "after restore")
    _append(g, o, kx[:, :, :5], vx[:, :, :5], blocks)
    _assert_same(g, o, "append after restore")
    # the snapshot is unchanged by all of it: restore it again
    rbq.restore_caches([g], gs)
    O.restore([o], os_)
    _assert_same(g, o, "second restore")


def test_restore_into_smaller_and_empty_caches(rot, blocks):
    k, v = _tokens(43, 1, 2, 300)
    src = rbq.RotatedQuantKVCache(1, 2, device=dev, rot=rot)
    osrc = O.QuantKVCache()
    _append(src, osrc, k, v, blocks)
    snap, osnap = src.snapshot(), O.snapshot([osrc])
    # a cache with 10 rows in a 256-row buffer: new buffers of exactly 300 rows
    g = rbq.RotatedQuantKVCache(1, 2, device=dev, rot=rot)
    o = O.QuantKVCache()
    _append(g, o, k[:, :, :10], v[:, :, :10], blocks)
    g.restore(snap)
    O.restore([o], osnap)
    assert g.capacity == 300
    _assert_same(g, o, "restore into a smaller cache")
    kx, vx = _tokens(44, 1, 2, 3)
    _append(g, o, kx, vx, blocks)
    assert g.capacity == o.capacity == 556
    _assert_same(g, o, "append after growth from a restored buffer")
    # empty marker: a cache without rows
    e = rbq.RotatedQuantKVCache(1, 2, device=dev, rot=rot)
    esnap, oesnap = e.snapshot(), O.snapshot([O.QuantKVCache()])
    assert esnap.desc is None and esnap.offset == 0
    g.restore(esnap)
    O.restore([o], oesnap)
    assert g.arrays is None and g.offset == 0 and g.capacity == 0
    _append(g, o, k[:, :, :7], v[:, :, :7], blocks)
    _assert_same(g, o, "append after restoring the empty marker")
    with pytest.raises(ValueError):
        g.restore(rbq.CacheSnapshot(None, None, ("64", "8", "3")))


def test_commit_verified_snapshot_matches_oracle(rot, blocks):
    k, v = _tokens(45, 1, 2, 40)
    g = rbq.RotatedQuantKVCache(1, 2, device=dev, rot=rot)
    o = O.QuantKVCache()
    _append(g, o, k[:, :, :37], v[:, :, :37], blocks)
    gsn, osn = [], []
    for i in range(3):
        _append(g, o, k[:, :, 37 + i:38 + i], v[:, :, 37 + i:38 + i], blocks)
        gsn.append(rbq.snapshot_caches([g]))
        osn.append(O.snapshot([o]))
    for acc, ver in ((3, 3), (0, None), (4, None)):
        assert rbq.commit_verified_snapshot([g], gsn, acc, ver) == \
            O.commit_verified_snapshot([o], osn, acc, ver)
        _assert_same(g, o, f"commit accepted={acc} verified={ver}")
    assert rbq.commit_verified_snapshot([g], gsn, 2, 3) is True
    assert O.commit_verified_snapshot([o], osn, 2, 3) is True
    _assert_same(g, o, "commit accepted=2 verified=3")
    assert g.offset == 39


def _raw_cache(B, H, cap, off, dtype=torch.bfloat16, seed=0):
    """A descriptor over random device buffers (any capacity, no rows meaning)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    arrs = {}
    for name, w in (("k_words", 32), ("k_scales", 2), ("k_biases", 2), ("v_words", 24),
                    ("v_scales", 2), ("v_biases", 2)):
        arrs[name] = torch.randint(-2**31, 2**31 - 1, (B, H, cap, w), dtype=torch.int32,
                                   generator=gen).to(dev)
    d = capi.rbq_kv_cache(B=B, H_kv=H, head_dim=256, group_size=64, k_bits=4, v_bits=3,
                          dtype=capi.DTYPE_CODES[dtype], flags=0, capacity=cap, offset=off)
    for name, t in arrs.items():
        setattr(d, name, t.data_ptr())
    return d, arrs


@pytest.mark.parametrize("B,H,src_cap,dst_cap,n", [
    (1, 1, 1, 1, 1), (2, 2, 301, 257, 257), (3, 2, 999, 1001, 997), (1, 2, 4096, 4097, 4095),
    (2, 1, 300, 300, 0)])
def test_prefix_copy_bit_exact_any_capacity(B, H, src_cap, dst_cap, n):
    print(f"prefix copy B={B} H={H} caps {src_cap}->{dst_cap} n={n}", flush=True)
    s, sa = _raw_cache(B, H, src_cap, n, seed=1)
    d, da = _raw_cache(B, H, dst_cap, 0, seed=2)
    before = {k: t.clone() for k, t in da.items()}
    capi.rbq_kv_copy_prefix(s, d)
    torch.cuda.synchronize()
    assert d.offset == n
    for name in sa:
        assert torch.equal(da[name][:, :, :n], sa[name][:, :, :n]), name
        assert torch.equal(da[name][:, :, n:], before[name][:, :, n:]), name


def test_prefix_copy_at_batched_decode_size():
    w = W.WORKLOADS[3]
    print(f"prefix copy at {w.name} size", flush=True)
    s, sa = _raw_cache(w.B, w.Hkv, w.T + 256, w.T, seed=3)
    d, da = _raw_cache(w.B, w.Hkv, w.T, 0, seed=4)
    capi.rbq_kv_copy_prefix(s, d)
    torch.cuda.synchronize()
    for name in sa:
        assert torch.equal(da[name], sa[name][:, :, :w.T]), name


def test_prefix_copy_errors():
    s, _ = _raw_cache(1, 2, 64, 64, seed=5)
    d, _ = _raw_cache(1, 2, 32, 0, seed=6)
    with pytest.raises(capi.RbqError):
        capi.rbq_kv_copy_prefix(s, d)  # destination too small
    assert d.offset == 0
    with pytest.raises(capi.RbqError):
        capi.rbq_kv_copy_prefix(s, s)  # overlapping arrays

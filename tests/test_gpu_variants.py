"""GPU parity of the configuration variants through the C ABI: head_dim 64 /
128 / 256, group 32 / 64 / 128, K and V widths 2-8, the two-sided rotation
and the page's own rotation precision (packed words, scales and biases bit
for bit against the oracle; attention within 2e-3), the general tile
attention kernel on long query blocks (prefill-length L) for the default
configuration, masks and key splits on the tile kernel, and the prefix copy
of variant caches.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O

pytestmark = pytest.mark.gpu

ATOL = 2e-3
rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402

NAMES = (("k_words", "kw"), ("k_scales", "ks"), ("k_biases", "kb"),
         ("v_words", "vw"), ("v_scales", "vs"), ("v_biases", "vb"))

# head_dim, group, k_bits, v_bits, dtype, two-sided rotation, round_rotated
VARIANTS = [
    (64, 32, 2, 8, "f16", False, False),
    (128, 64, 5, 6, "bf16", True, False),
    (256, 128, 8, 2, "bf16", False, True),
    (128, 128, 3, 4, "f16", False, True),
    (256, 32, 6, 5, "bf16", True, False),
    (64, 64, 4, 3, "bf16", False, False),
    (256, 64, 4, 3, "bf16", True, True),   # default sizes, dedicated kernels, both options
    (128, 32, 4, 4, "bf16", False, False),
    (256, 64, 4, 4, "f16", True, False),   # head_dim 256, 4 groups: paired single-wave rows up to 8 rows
    (256, 64, 4, 3, "f16", False, True),
]


def _vid(v):
    return "D{}_g{}_k{}v{}_{}{}{}".format(v[0], v[1], v[2], v[3], v[4], "_2s" if v[5] else "",
                                         "_rr" if v[6] else "")


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def _setup(var, dev, B, Hkv, T, seed, chunks=(0.6,)):
    D, gs, kb, vb, dtype, two, rr = var
    tdt = W._TORCH_DTYPES[dtype]
    draws = W.rotation_draws(seed, D)
    blocks = O.rotation_blocks(draws, mode="two_sided" if two else "printed")
    if rr:
        blocks = O.round_to_dtype(blocks, dtype)
    rot = rbq.build_block_so4(D, seed, dev, two_sided=two, round_to=tdt if rr else None)
    np.testing.assert_array_equal(rot.cpu().numpy(), blocks)
    c = rbq.RotatedQuantKVCache(B, Hkv, dtype=tdt, device=dev, rot=rot, head_dim=D,
                                group_size=gs, k_bits=kb, v_bits=vb, round_rotated=rr)
    oc = O.QuantKVCache(k_bits=kb, v_bits=vb, dtype=dtype, group=gs, round_rotated=rr)
    k = W.random_rows([seed, 1], (B, Hkv, T, D), dtype, "student_t3")
    v = W.random_rows([seed, 2], (B, Hkv, T, D), dtype)
    cut = [0] + [int(f * T) for f in chunks] + [T]
    for a, b in zip(cut[:-1], cut[1:]):
        c.append(k[:, :, a:b].contiguous().to(dev), v[:, :, a:b].contiguous().to(dev))
        oc.append(k[:, :, a:b].float().numpy(), v[:, :, a:b].float().numpy(), blocks)
    return c, oc, blocks, rot


def _assert_cache_equal(c, oc):
    torch.cuda.synchronize()
    assert (c.offset, c.capacity) == (oc.offset, oc.capacity)
    rows = c.rows()
    for name, oname in NAMES:
        got = rows[name].cpu()
        got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
        ref = oc.arrays[oname][:, :, :oc.offset]
        assert got.shape == ref.shape, name
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("var", VARIANTS, ids=_vid)
def test_variant_append_bit_exact(var, dev):
    print(f"[variant append] {_vid(var)}", flush=True)
    c, oc, _, _ = _setup(var, dev, 2, 2, 301, 11, chunks=(0.3, 0.61))
    _assert_cache_equal(c, oc)


@pytest.mark.parametrize("var", VARIANTS, ids=_vid)
def test_variant_attention(var, dev):
    print(f"[variant attention] {_vid(var)}", flush=True)
    D = var[0]
    B, Hq, Hkv, T = 2, 8, 2, 333
    c, oc, blocks, _ = _setup(var, dev, B, Hkv, T, 12)
    for L, causal in ((1, True), (3, True), (5, False)):
        q = W.random_rows([13, L], (B, Hq, L, D), var[4])
        out = c.attend(q.to(dev), scale=D ** -0.5, causal=causal)
        torch.cuda.synchronize()
        ref = O.attention(q.float().numpy(), oc, D ** -0.5, causal, blocks)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= ATOL, (L, causal, err)


@pytest.mark.parametrize("var", [(256, 64, 4, 3, "bf16", False, False),
                                 (256, 64, 4, 4, "bf16", False, False)], ids=_vid)
@pytest.mark.parametrize("L", [70, 129])
def test_long_query_blocks(L, var, dev):
    # prefill-length query blocks: G = 8 L rows per kv head (the default
    # configuration in 8-row blocks of the dedicated kernel; K4/V4 in 64-row
    # blocks of the tile kernel, a ragged last one)
    print(f"[long block] {_vid(var)} L={L}", flush=True)
    B, Hq, Hkv, T = 1, 16, 2, 700
    c, oc, blocks, _ = _setup(var, dev, B, Hkv, T, 14)
    q = W.random_rows([15, L], (B, Hq, L, 256), "bf16")
    out = c.attend(q.to(dev), scale=1 / 16, causal=True)
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 1 / 16, True, blocks)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= ATOL, err
    # row 0 of the block is an L = 1 decode over the keys it sees (a call of
    # another shape, which rounds differently: both within the tolerance of
    # the oracle)
    c.trim(L - 1)
    oc.trim(L - 1)
    q1 = q[:, :, :1].contiguous()
    out1 = c.attend(q1.to(dev), scale=1 / 16, causal=True)
    torch.cuda.synchronize()
    ref1 = O.attention(q1.float().numpy(), oc, 1 / 16, True, blocks)
    np.testing.assert_allclose(ref1, ref[:, :, :1], rtol=0, atol=1e-9)
    err1 = float(np.abs(out1.cpu().numpy() - ref1).max())
    cross = float(np.abs(out1.cpu().numpy() - out[:, :, :1].cpu().numpy()).max())
    print(f"block error {err:.2e}, decode of row 0 {err1:.2e}, between them {cross:.2e}")
    assert err1 <= ATOL and cross <= ATOL


def test_tile_kernel_splits_agree(dev):
    var = (128, 64, 5, 6, "bf16", True, False)
    B, Hq, Hkv, T, L = 1, 4, 1, 2000, 2
    c, oc, blocks, _ = _setup(var, dev, B, Hkv, T, 16)
    q = W.random_rows([17, L], (B, Hq, L, 128), "bf16").to(dev)
    outs = []
    for S in (1, 3, 7, 63):
        outs.append(c.attend(q, scale=128 ** -0.5, causal=True, splits=S))
    torch.cuda.synchronize()
    ref = O.attention(q.cpu().float().numpy(), oc, 128 ** -0.5, True, blocks)
    for o in outs:
        assert float(np.abs(o.cpu().numpy() - ref).max()) <= ATOL
        assert float(np.abs(o.cpu().numpy() - outs[0].cpu().numpy()).max()) <= 1e-5


@pytest.mark.parametrize("kind", ["bool", "f32", "dtype"])
def test_tile_kernel_masks(kind, dev):
    var = (64, 32, 2, 8, "f16", False, False)
    B, Hq, Hkv, T, L = 2, 4, 2, 200, 3
    c, oc, blocks, _ = _setup(var, dev, B, Hkv, T, 18)
    q = W.random_rows([19, L], (B, Hq, L, 64), "f16")
    g = np.random.default_rng(20)
    if kind == "bool":
        m = g.random((B, 1, L, T)) < 0.7
        m[..., 0] = True
        mask = torch.from_numpy(m)
        ref_mask = m
    else:
        m = (g.standard_normal((1, Hq, L, T)) * 2).astype(np.float32)
        mask = torch.from_numpy(m).to(torch.float16 if kind == "dtype" else torch.float32)
        ref_mask = mask.float().numpy().astype(np.float64)
    out = c.attend(q.to(dev), scale=0.125, causal=True, mask=mask.to(dev))
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 0.125, True, blocks, mask=ref_mask)
    assert float(np.abs(out.cpu().numpy() - ref).max()) <= ATOL


@pytest.mark.parametrize("var", [VARIANTS[0], VARIANTS[5], VARIANTS[2]], ids=_vid)
def test_variant_snapshot_restore_and_tile(var, dev):
    # prefix copies move 16-bit units: one-group rows (head_dim 64, group 64)
    # are 2 bytes per scale row
    c, oc, _, _ = _setup(var, dev, 2, 1, 77, 21)
    snap = c.snapshot()
    k = W.random_rows([22, 1], (2, 1, 5, var[0]), var[4]).to(dev)
    c.append(k, k)
    c.restore(snap)
    _assert_cache_equal(c, oc)
    c1, oc1, _, _ = _setup(var, dev, 1, 2, 45, 23)
    c1.tile(3)
    O.tile_cache(oc1, 3)
    torch.cuda.synchronize()
    rows = c1.rows()
    for name, oname in NAMES:
        got = rows[name].cpu()
        got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
        np.testing.assert_array_equal(got, oc1.arrays[oname][:, :, :oc1.offset])


@pytest.mark.parametrize("var", [VARIANTS[3], VARIANTS[5], VARIANTS[1]], ids=_vid)
def test_tile_kernel_exact_capacity_cache(var, dev):
    # A cache restored from a snapshot into fresh buffers holds exactly
    # `offset` rows (odd here): the slabs of the six arrays are not 16-byte
    # aligned and the last key row ends the buffer, so the tile transfers take
    # their 4-byte path and must not read past row T - 1.
    D = var[0]
    B, Hq, Hkv, T = 2, 8, 2, 257
    c, oc, blocks, rot = _setup(var, dev, B, Hkv, T, 24)
    snap = c.snapshot()
    e = rbq.RotatedQuantKVCache(B, Hkv, dtype=W._TORCH_DTYPES[var[4]], device=dev, rot=rot,
                                head_dim=D, group_size=var[1], k_bits=var[2], v_bits=var[3],
                                round_rotated=var[6])
    e.restore(snap)
    assert e.capacity == e.offset == T
    for L in (1, 3, 17):
        q = W.random_rows([25, L], (B, Hq, L, D), var[4])
        out = e.attend(q.to(dev), scale=D ** -0.5, causal=True)
        torch.cuda.synchronize()
        ref = O.attention(q.float().numpy(), oc, D ** -0.5, True, blocks)
        assert float(np.abs(out.cpu().numpy() - ref).max()) <= ATOL, L


def test_tile_kernel_full_prefill_block(dev):
    # L = offset: every cached row is a query row (row 0 sees one key); four-wave
    # blocks with a ragged last block
    var = (128, 32, 3, 5, "bf16", True, False)
    B, Hq, Hkv, T = 1, 4, 2, 100
    c, oc, blocks, _ = _setup(var, dev, B, Hkv, T, 26)
    q = W.random_rows([27, T], (B, Hq, T, 128), "bf16")
    out = c.attend(q.to(dev), scale=128 ** -0.5, causal=True)
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 128 ** -0.5, True, blocks)
    assert float(np.abs(out.cpu().numpy() - ref).max()) <= ATOL


@pytest.mark.parametrize("splits", [1, 4])
def test_tile_kernel_four_wave_mask_and_splits(splits, dev):
    # 24 query rows per kv head (four-wave blocks) with a boolean tree-like mask
    var = (128, 64, 4, 3, "f16", False, False)
    B, Hq, Hkv, T, L = 2, 8, 2, 500, 6
    c, oc, blocks, _ = _setup(var, dev, B, Hkv, T, 28)
    q = W.random_rows([29, L], (B, Hq, L, 128), "f16")
    keep = np.ones((1, 1, L, T), bool)
    keep[..., T - L:] = np.tril(np.ones((L, L), bool))
    keep[..., 0, T - L + 3:] = False
    keep[..., 2, T - L + 1] = False
    out = c.attend(q.to(dev), scale=128 ** -0.5, causal=False, mask=torch.from_numpy(keep).to(dev),
                   splits=splits)
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 128 ** -0.5, False, blocks, mask=keep)
    assert float(np.abs(out.cpu().numpy() - ref).max()) <= ATOL


@pytest.mark.parametrize("var", [VARIANTS[0], VARIANTS[4]], ids=_vid)
def test_tile_kernel_single_key(var, dev):
    # one cached row: the output is that row's dequantised V, rotated back
    D = var[0]
    c, oc, blocks, _ = _setup(var, dev, 1, 1, 1, 30, chunks=())
    q = W.random_rows([31, 1], (1, 2, 1, D), var[4])
    out = c.attend(q.to(dev), scale=D ** -0.5, causal=True)
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, D ** -0.5, True, blocks)
    vhat = O.inverse_rotate(oc.dequant_kv(0, 0)[1][0].astype(np.float32), blocks)
    np.testing.assert_allclose(ref[0, 0, 0], vhat, rtol=0, atol=1e-6)
    assert float(np.abs(out.cpu().numpy() - ref).max()) <= ATOL


# single-wave tile workgroups (up to 16 rows per kv head at head_dim <= 128,
# and at head_dim 256 with 8 groups per row; up to 8 rows, paired hi / lo
# operand rows, at head_dim 256 with 2 and 4 groups) with one split, so that
# each workgroup walks many tiles (the running scale powers and the staging
# transfers are carried across all of them): 4 groups per row (two scale /
# bias items per thread), 2 and 8; at head_dim 256 with 2 or 4 groups, L = 2
# (16 rows) runs the four-wave shape over the same keys
@pytest.mark.parametrize("var", [(128, 32, 4, 4, "bf16", False, False),
                                 (128, 32, 3, 5, "f16", True, False),
                                 (128, 64, 4, 4, "bf16", True, False),
                                 (256, 32, 4, 4, "bf16", False, False),
                                 (256, 32, 6, 2, "f16", True, False),
                                 (256, 64, 4, 4, "f16", True, False),
                                 (256, 64, 5, 2, "bf16", False, False),
                                 (256, 128, 4, 3, "bf16", True, False)], ids=_vid)
@pytest.mark.parametrize("splits", [1, 2])
def test_single_wave_tile_kernel_many_tiles(var, splits, dev):
    print(f"[single-wave tiles] {_vid(var)} splits={splits}", flush=True)
    D = var[0]
    B, Hq, Hkv, T = 1, 16, 2, 2900   # 91 tiles of 32 keys per split at splits=1
    c, oc, blocks, _ = _setup(var, dev, B, Hkv, T, 32)
    assert capi.rbq_quant_attn_splits(c.desc, Hq, 1) >= 1
    for L in (1, 2):
        q = W.random_rows([33, L], (B, Hq, L, D), var[4])
        out = c.attend(q.to(dev), scale=D ** -0.5, causal=True, splits=splits)
        torch.cuda.synchronize()
        ref = O.attention(q.float().numpy(), oc, D ** -0.5, True, blocks)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= ATOL, (L, err)

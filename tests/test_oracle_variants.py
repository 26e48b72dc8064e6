"""Pins of the oracle's variants beyond the default K4/V3, group-64,
head_dim-256 configuration (CPU only).

Sources: the page "mlx_streaming/core/cache/quant_kv.py": the width list of
``_packed_words`` (2/3/4/5/6/8 bits), the cache constructor's ``group_size``,
``build_block_so4`` for any head_dim divisible by 4, the ``_quat_right_conj``
docstring (a right multiplication by conj(q): the two-sided rotation), and
``rotate_last`` (``x @ R.astype(x.dtype)``: the page's own precision).  Each
check compares with something other than the oracle: the Hamilton product
written out in this file, closed forms, brute-force loops, torch.
"""
import numpy as np
import pytest
import torch

from oracle import brute
from oracle import rbq_oracle as O
import workloads as W

RNG = np.random.default_rng(4321)
WIDTHS = [2, 3, 4, 5, 6, 8]


def qmul(p, q):
    """Hamilton product written out from i^2 = j^2 = k^2 = ijk = -1."""
    a1, b1, c1, d1 = p
    a2, b2, c2, d2 = q
    return np.array([a1 * a2 - b1 * b2 - c1 * c2 - d1 * d2,
                     a1 * b2 + b1 * a2 + c1 * d2 - d1 * c2,
                     a1 * c2 - b1 * d2 + c1 * a2 + d1 * b2,
                     a1 * d2 + b1 * c2 - c1 * b2 + d1 * a2])


def conj(q):
    return np.array([q[0], -q[1], -q[2], -q[3]])


def unit(v):
    v = np.asarray(v, np.float64)
    return v / np.linalg.norm(v)


# ------------------------------------------------------- two-sided rotation --

def test_true_right_conj_is_right_multiplication():
    # The _quat_right_conj docstring: v -> v * conj(q).
    for _ in range(20):
        q = unit(RNG.standard_normal(4))
        v = RNG.standard_normal(4)
        np.testing.assert_allclose(O.quat_right_true_conj(q) @ v, qmul(v, conj(q)), atol=1e-14)


def test_two_sided_block_is_left_times_right_multiplication():
    # Two-sided block: v -> qL * v * conj(qR) (column-vector form), for every draw.
    draws = W.rotation_draws(5, 128)
    blocks = O.rotation_blocks(draws, mode="two_sided")
    assert blocks.shape == (32, 4, 4)
    for b in range(32):
        qL, qR = unit(draws[b, 0]), unit(draws[b, 1])
        for _ in range(3):
            v = RNG.standard_normal(4)
            ref = qmul(qmul(qL, v), conj(qR))
            assert np.abs(blocks[b].astype(np.float64) @ v - ref).max() <= 4e-7 * np.abs(v).sum()


def test_two_sided_blocks_orthogonal_det_one_and_differ_from_printed():
    draws = W.rotation_draws(0, 256)
    two = O.rotation_blocks(draws, mode="two_sided").astype(np.float64)
    printed = O.rotation_blocks(draws).astype(np.float64)
    for B in two:
        assert np.abs(B @ B.T - np.eye(4)).max() <= 1e-6
        assert abs(np.linalg.det(B) - 1.0) <= 1e-6
    assert np.abs(two - printed).max() > 0.1


def test_two_sided_equal_draws_fix_the_real_axis():
    # q * 1 * conj(q) = 1: with equal draws the block maps e0 to e0 and is a
    # rotation of the 3-D imaginary part (not the identity, unlike the
    # printed form).
    d = RNG.standard_normal((6, 4)).astype(np.float32)
    blocks = O.rotation_blocks(np.stack([d, d], axis=1), mode="two_sided").astype(np.float64)
    for B in blocks:
        np.testing.assert_allclose(B[:, 0], [1, 0, 0, 0], atol=2e-7)
        np.testing.assert_allclose(B[0, :], [1, 0, 0, 0], atol=2e-7)
        assert np.abs(B - np.eye(4)).max() > 1e-3


def test_two_sided_reaches_right_isoclinic_rotations():
    # With qL = 1 the block is a pure right multiplication, which no printed
    # block (a left multiplication) equals unless it is +-I.
    qR = RNG.standard_normal(4).astype(np.float32)
    draws = np.stack([np.array([[1, 0, 0, 0]], np.float32), qR[None]], axis=1)
    B = O.rotation_blocks(draws, mode="two_sided")[0].astype(np.float64)
    np.testing.assert_allclose(B, O.quat_right_true_conj(unit(qR)), atol=1e-7)
    # a left multiplication matrix L(p) has the structure of quat_left; B does not
    p = B[:, 0]
    assert np.abs(B - O.quat_left(p)).max() > 1e-3


# ------------------------------------------------ the page's own precision --

@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_round_rotated_matches_torch_low_precision_matmul(dtype):
    # rotate_last computes x @ R.astype(x.dtype) in the input dtype: torch's
    # CPU matmul of the dtype-rounded operands (dense M, zeros elsewhere).
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    blocks = O.round_to_dtype(O.rotation_blocks(W.rotation_draws(0, 256)), dtype)
    x = W.random_rows(21, (64, 256), dtype)
    got = O.rotate_for_cache(x.float().numpy(), blocks, dtype, round_rotated=True)
    M = torch.from_numpy(O.dense_rotation(blocks)).to(tdt)
    ref = (x.to(tdt) @ M).float().numpy()
    same = got == ref
    assert same.mean() >= 0.995
    # where fp32 accumulation order differs, at most one unit in the last place
    mant = 7 if dtype == "bf16" else 10
    e = np.floor(np.log2(np.maximum(np.abs(ref).astype(np.float64), 2.0 ** -14)))
    ulp = 2.0 ** (e - mant)
    assert np.all(np.abs(got - ref)[~same] <= ulp[~same])


def test_round_rotated_values_are_dtype_values_and_default_is_not():
    blocks = O.rotation_blocks(W.rotation_draws(0, 256))
    x = W.random_rows(22, (8, 256), "bf16").float().numpy()
    r = O.rotate_for_cache(x, O.round_to_dtype(blocks, "bf16"), "bf16", True)
    np.testing.assert_array_equal(r, O.round_to_dtype(r, "bf16"))
    d = O.rotate_for_cache(x, blocks, "bf16", False)
    assert np.any(d != O.round_to_dtype(d, "bf16"))
    np.testing.assert_array_equal(d, O.rotate(x, blocks))


# ------------------------------------------------------ widths and groups --

@pytest.mark.parametrize("group", [32, 64, 128])
@pytest.mark.parametrize("bits", WIDTHS)
def test_exact_grid_group_all_widths(bits, group):
    # A row on the grid beta0 + k/4, k = 0..2^bits-1 repeated, every group
    # holding the whole grid (group >= 2^bits, or the grid cut to the group):
    # scale 1/4, codes k, exact dequantisation.
    levels = min(2 ** bits, group)
    row = np.array([-2.0 + (j % levels) / 4.0 for j in range(256)], np.float32)
    codes, s, b = O.quantize(row, bits, "bf16", group)
    expect_s = (levels - 1) / 4.0 / (2 ** bits - 1)
    np.testing.assert_array_equal(s, O.round_to_dtype(np.full(256 // group, expect_s, np.float32), "bf16"))
    np.testing.assert_array_equal(b, np.full(256 // group, -2.0, np.float32))
    if levels == 2 ** bits:
        np.testing.assert_array_equal(codes, np.arange(256) % levels)
        np.testing.assert_array_equal(O.dequantize(codes, s, b, group), row.astype(np.float64))


@pytest.mark.parametrize("group", [32, 128])
@pytest.mark.parametrize("bits", WIDTHS)
def test_error_bound_all_widths(bits, group):
    # |y - x_hat| <= s/2 (up to the fp32 rounding of the division) for values
    # that the clip leaves alone; codes in range, group min -> 0, max -> top.
    x = W.random_rows(23, (64, 256), "bf16", dist="student_t3").float().numpy()
    y = O.rotate(x, O.rotation_blocks(W.rotation_draws(0, 256)))
    codes, s, b = O.quantize(y, bits, "bf16", group)
    top = 2 ** bits - 1
    assert codes.max() <= top
    yg = y.reshape(-1, 256 // group, group).astype(np.float64)
    xh = O.dequantize(codes, s, b, group).reshape(yg.shape)
    s64 = s.astype(np.float64)[..., None]
    raw = (yg - b.astype(np.float64)[..., None]) / s64
    inside = (raw > -0.5) & (raw < top + 0.5)
    assert inside.mean() > 0.99
    assert np.all(np.abs(xh - yg)[inside] <= np.broadcast_to(s64 / 2, yg.shape)[inside] * (1 + 2.0 ** -19))
    cg = codes.reshape(yg.shape)
    ok = np.abs(b.astype(np.float64) - yg.min(-1)) < s.astype(np.float64) / 2
    amin = np.take_along_axis(cg, yg.argmin(-1)[..., None], -1)[..., 0]
    amax = np.take_along_axis(cg, yg.argmax(-1)[..., None], -1)[..., 0]
    assert np.all(amin[ok] == 0)
    # the max reaches the top code unless the scale's rounding to bf16 (up to
    # 2^-9 relative) moves it by half a step or more: only possible at 8 bits
    # (255 * 2^-9 + the bias rounding can exceed 1/2)
    if bits <= 6:
        assert np.all(amax[ok] == top)
    else:
        assert np.all(amax[ok] >= top - 1) and np.mean(amax[ok] == top) > 0.5


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bits,group,D", [(2, 32, 64), (5, 64, 128), (6, 128, 128), (8, 32, 256),
                                          (3, 128, 256)])
def test_quantize_pack_matches_brute(bits, group, D, dtype):
    x = W.random_rows(24, (4, D), dtype, dist="student_t3").float().numpy()
    blocks = O.rotation_blocks(W.rotation_draws(1, D))
    words, s, b = O.quantize_rows(x, blocks, bits, dtype, group)
    assert words.shape == (4, D * bits // 32)
    for r in range(4):
        y = brute.rotate_row(x[r].tolist(), blocks.tolist())
        bc, bs, bb = brute.quantize_row(y, bits, dtype, group)
        assert words[r].tolist() == brute.pack_row(bc, bits)
        assert s[r].tolist() == bs and b[r].tolist() == bb


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bits", WIDTHS)
def test_pack_roundtrip_other_head_dims(bits, D):
    codes = RNG.integers(0, 2 ** bits, size=(3, D))
    words = O.pack(codes, bits)
    assert words.shape == (3, D * bits // 32)
    for r in range(3):
        assert words[r].tolist() == brute.pack_row(codes[r].tolist(), bits)
    np.testing.assert_array_equal(O.unpack(words, bits, D), codes)


def test_cache_variant_arrays_and_meta_state():
    # _init_quant: words dim*bits//32, dim/group scales and biases per row.
    c = O.QuantKVCache(k_bits=5, v_bits=2, dtype="f16", group=32)
    k = W.random_rows(25, (1, 2, 10, 128), "f16").float().numpy()
    c.append(k, k, None)
    a = c.arrays
    assert a["kw"].shape == (1, 2, 256, 20) and a["vw"].shape == (1, 2, 256, 8)
    assert a["ks"].shape == (1, 2, 256, 4) and a["vb"].shape == (1, 2, 256, 4)
    assert O.meta_state(c) == ("32", "5", "2")
    kh, vh = c.dequant_kv(0, 1)
    for t in range(10):
        bc, bs, bb = brute.quantize_row(k[0, 1, t].tolist(), 5, "f16", 32)
        assert kh[t].tolist() == brute.dequant_row(bc, bs, bb, 32)


def test_round_rotated_cache_quantizes_rounded_rows():
    blocks = O.round_to_dtype(O.rotation_blocks(W.rotation_draws(0, 128)), "bf16")
    x = W.random_rows(26, (1, 1, 5, 128), "bf16").float().numpy()
    c = O.QuantKVCache(k_bits=4, v_bits=4, group=64, round_rotated=True)
    c.append(x, x, blocks)
    for t in range(5):
        y = [brute.bf16(v) for v in brute.rotate_row(x[0, 0, t].tolist(), blocks.tolist())]
        bc, bs, bb = brute.quantize_row(y, 4, "bf16", 64)
        assert c.arrays["kw"][0, 0, t].tolist() == brute.pack_row(bc, 4)


# --------------------------------------------------------------- attention --

@pytest.mark.parametrize("kb,vb,group,D,mode", [(2, 8, 32, 64, "printed"), (5, 6, 64, 128, "two_sided"),
                                                (8, 2, 128, 256, "two_sided"), (3, 5, 32, 128, "printed")])
def test_variant_attention_matches_brute(kb, vb, group, D, mode):
    blocks = O.rotation_blocks(W.rotation_draws(2, D), mode=mode)
    B, Hq, Hkv, T, L = 1, 4, 2, 29, 3
    c = O.QuantKVCache(k_bits=kb, v_bits=vb, group=group)
    k = W.random_rows(27, (B, Hkv, T, D), "bf16").float().numpy()
    v = W.random_rows(28, (B, Hkv, T, D), "bf16").float().numpy()
    c.append(k, v, blocks)
    q = W.random_rows(29, (B, Hq, L, D), "bf16").float().numpy()
    scale = D ** -0.5
    out = O.attention(q, c, scale, True, blocks)
    for h in range(Hq):
        kh, vh = c.dequant_kv(0, h // 2)
        for i in range(L):
            ref = brute.attention_row(q[0, h, i].tolist(), kh.tolist(), vh.tolist(), T - L + i + 1,
                                      scale, blocks.tolist())
            np.testing.assert_allclose(out[0, h, i], ref, rtol=0, atol=1e-6)


def test_variant_attention_rotation_cancels():
    # With the two-sided rotation as well: attention over the rotated cache,
    # rotated back, equals attention of the unrotated q over the dequantised
    # rows rotated back (q.k and the output are invariant under M).
    D = 128
    blocks = O.rotation_blocks(W.rotation_draws(3, D), mode="two_sided")
    c = O.QuantKVCache(k_bits=6, v_bits=5, group=64)
    k = W.random_rows(30, (1, 1, 40, D), "bf16").float().numpy()
    c.append(k, k, blocks)
    q = W.random_rows(31, (1, 1, 1, D), "bf16").float().numpy()
    out = O.attention(q, c, D ** -0.5, False, blocks)[0, 0, 0]
    Minv = O.dense_rotation(blocks).T
    kh, vh = c.dequant_kv(0, 0)
    sc = (kh @ Minv) @ q[0, 0, 0].astype(np.float64) * D ** -0.5
    p = np.exp(sc - sc.max())
    ref = (p @ (vh @ Minv)) / p.sum()
    np.testing.assert_allclose(out, ref, rtol=0, atol=2e-6)

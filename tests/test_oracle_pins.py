"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it checks and where the fact comes from: the pages
("quant_kv.py": rotation, cache, SDPA sections; "mtp/kv_cache.py":
commit_verified_prefix), closed forms, special cases, invariants, brute force
on tiny inputs, or an independent library routine (torch, numpy.linalg).
"""
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import rbq_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------- helpers --

# Quaternion basis products from i^2 = j^2 = k^2 = ijk = -1, written as a table
# (sign, index) for e_a * e_b with e_0 = 1, e_1 = i, e_2 = j, e_3 = k.
_QTABLE = {
    (0, 0): (1, 0), (0, 1): (1, 1), (0, 2): (1, 2), (0, 3): (1, 3),
    (1, 0): (1, 1), (1, 1): (-1, 0), (1, 2): (1, 3), (1, 3): (-1, 2),
    (2, 0): (1, 2), (2, 1): (-1, 3), (2, 2): (-1, 0), (2, 3): (1, 1),
    (3, 0): (1, 3), (3, 1): (1, 2), (3, 2): (-1, 1), (3, 3): (-1, 0),
}


def qmul(p, q):
    out = [0.0] * 4
    for a in range(4):
        for b in range(4):
            s, k = _QTABLE[(a, b)]
            out[k] += s * p[a] * q[b]
    return np.array(out)


def conj(q):
    return np.array([q[0], -q[1], -q[2], -q[3]])


def unit(v):
    v = np.asarray(v, np.float64)
    return v / np.linalg.norm(v)


def left_matrix_from_table(p):
    """Matrix of v -> p*v built column by column from the basis table."""
    return np.stack([qmul(p, np.eye(4)[j]) for j in range(4)], axis=1)


def seed0_blocks():
    return O.rotation_blocks(W.rotation_draws(0, 256))


# --------------------------------------------------------------- rotation --

def test_quat_left_is_left_multiplication():
    # quant_kv.py, _quat_left: L(q) v = q * v (Hamilton product).
    for _ in range(20):
        q = unit(RNG.standard_normal(4))
        v = RNG.standard_normal(4)
        np.testing.assert_allclose(O.quat_left(q) @ v, qmul(q, v), atol=1e-14)


def test_quat_right_conj_as_printed_is_left_mult_by_conj():
    # Reading R1: the printed _quat_right_conj entries give v -> conj(q) * v,
    # i.e. L(q)^T, and not the docstring's v -> v * conj(q).
    diffs = []
    for _ in range(20):
        q = unit(RNG.standard_normal(4))
        v = RNG.standard_normal(4)
        R = O.quat_right_conj(q)
        np.testing.assert_allclose(R @ v, qmul(conj(q), v), atol=1e-14)
        np.testing.assert_array_equal(R, O.quat_left(q).T)
        diffs.append(np.abs(R @ v - qmul(v, conj(q))).max())
    assert max(diffs) > 1e-3  # the docstring's map is a different one


def test_block_equals_left_mult_by_product_quaternion():
    # build_block_so4: block = L(qL) R(conj qR) = L(qL * conj qR) (closed form).
    draws = W.rotation_draws(0, 256)
    blocks = O.rotation_blocks(draws)
    for b in range(64):
        qL = unit(draws[b, 0].astype(np.float64))
        qR = unit(draws[b, 1].astype(np.float64))
        ref = left_matrix_from_table(qmul(qL, conj(qR)))
        assert np.abs(blocks[b] - ref).max() <= 2e-7


def test_blocks_orthogonal_with_det_one():
    # Design notes of quant_kv.py: each block is an SO(4) rotation.
    blocks = seed0_blocks()
    for B in blocks.astype(np.float64):
        assert np.abs(B @ B.T - np.eye(4)).max() <= 1e-6
        assert abs(np.linalg.det(B) - 1.0) <= 1e-6


def test_equal_draws_give_identity():
    # L(q) L(q)^T = I for a unit q: equal left/right draws give the identity
    # (the docstring's two-sided reading would give a rotation fixing e0 instead).
    d = RNG.standard_normal((8, 4)).astype(np.float32)
    draws = np.stack([d, d], axis=1)
    blocks = O.rotation_blocks(draws)
    assert np.abs(blocks - np.eye(4, dtype=np.float32)).max() <= 1e-7


def test_draw_order_left_then_right():
    # build_block_so4 draws 4 normals for qL then 4 for qR, block by block.
    d = W.rotation_draws(0, 256)
    ref = np.random.default_rng(0).standard_normal(512).astype(np.float32)
    np.testing.assert_array_equal(d.reshape(-1), ref)


def test_block_build_close_to_float32_build():
    # Reading R2 (fp64 build, one rounding) differs from a float32 build of the
    # same definition by float32 rounding only.
    draws = W.rotation_draws(0, 256)
    blocks = O.rotation_blocks(draws)
    for b in range(64):
        qL = draws[b, 0] / np.linalg.norm(draws[b, 0])
        qR = draws[b, 1] / np.linalg.norm(draws[b, 1])
        f32 = (O.quat_left(qL).astype(np.float32) @ O.quat_right_conj(qR).astype(np.float32))
        assert np.abs(f32 - blocks[b]).max() <= 5e-7


def test_zero_draw_rejected():
    draws = np.zeros((1, 2, 4), np.float32)
    with pytest.raises(ValueError):
        O.rotation_blocks(draws)


def test_rotate_matches_dense_matmul_and_brute():
    # rotate_last: y = x @ M with M the dense block-diagonal matrix.
    blocks = seed0_blocks()
    M = O.dense_rotation(blocks)
    x = W.random_rows(7, (5, 256), "bf16").float().numpy()
    y = O.rotate(x, blocks)
    np.testing.assert_allclose(y, x.astype(np.float64) @ M, rtol=0, atol=2e-6)
    for r in range(2):
        assert brute.rotate_row(list(x[r]), blocks.tolist()) == y[r].tolist()
    z = O.inverse_rotate(y, blocks)
    np.testing.assert_allclose(z, y.astype(np.float64) @ M.T, rtol=0, atol=2e-6)
    for r in range(2):
        assert brute.inverse_rotate_row(list(y[r]), blocks.tolist()) == z[r].tolist()


def test_rotation_preserves_dot_products_and_inverts():
    # Design notes: q and k get the same rotation, so q.k^T is unchanged.
    blocks = seed0_blocks()
    q = W.random_rows(8, (16, 256), "f16").float().numpy().astype(np.float64)
    k = W.random_rows(9, (16, 256), "f16").float().numpy().astype(np.float64)
    qr = O.rotate(q, blocks).astype(np.float64)
    kr = O.rotate(k, blocks).astype(np.float64)
    lhs = (qr * kr).sum(-1)
    rhs = (q * k).sum(-1)
    bound = 1e-5 * np.linalg.norm(q, axis=-1) * np.linalg.norm(k, axis=-1)
    assert np.all(np.abs(lhs - rhs) <= bound)
    back = O.inverse_rotate(qr.astype(np.float32), blocks).astype(np.float64)
    assert np.all(np.abs(back - q).max(-1) <= 1e-6 * np.linalg.norm(q, axis=-1))


# -------------------------------------------------------------- quantizer --

def _tricky_f32(n):
    x = RNG.standard_normal(n).astype(np.float32) * np.float32(3)
    u = x.view(np.uint32)
    u[: n // 4] = (u[: n // 4] & 0xFFFF0000) | 0x8000        # exact bf16 ties
    u[n // 4: n // 2] = (u[n // 4: n // 2] & 0xFFFF0000) | 0x7FFF
    return u.view(np.float32)


def test_bf16_rounding_matches_torch():
    x = _tricky_f32(1 << 16)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(O.round_to_dtype(x, "bf16"), ref)
    for v in x[:200]:
        assert brute.bf16(float(v)) == float(O.round_to_dtype(np.array([v]), "bf16")[0])


def test_f16_rounding_matches_torch():
    x = (RNG.standard_normal(1 << 16) * 100).astype(np.float32)
    x[:100] = np.float32(1e-6) * np.arange(100, dtype=np.float32)      # subnormal halves
    ref = torch.from_numpy(x.copy()).to(torch.float16).float().numpy()
    np.testing.assert_array_equal(O.round_to_dtype(x, "f16"), ref)
    for v in x[:200]:
        assert brute.f16(float(v)) == float(O.round_to_dtype(np.array([v]), "f16")[0])


@pytest.mark.parametrize("bits", [4, 3])
def test_exact_grid_group(bits):
    # A group laid on the grid beta0 + k/4 (k = 0..2^bits-1): scale 1/4,
    # bias beta0, codes k, dequantisation exact.
    levels = 2 ** bits
    row = np.array([-2.0 + (j % levels) / 4.0 for j in range(256)], np.float32)
    for dtype in ("bf16", "f16"):
        codes, s, b = O.quantize(row, bits, dtype)
        np.testing.assert_array_equal(s, np.full(4, 0.25, np.float32))
        np.testing.assert_array_equal(b, np.full(4, -2.0, np.float32))
        np.testing.assert_array_equal(codes, np.arange(256) % levels)
        np.testing.assert_array_equal(O.dequantize(codes, s, b), row.astype(np.float64))


def test_round_half_even_ties():
    # Group holding 0 and 15 (scale 1, bias 0) and the ties 0.5, 1.5, 2.5, 3.5.
    g = np.full(64, 5.0, np.float32)
    g[0], g[1] = 0.0, 15.0
    g[2:6] = [0.5, 1.5, 2.5, 3.5]
    row = np.tile(g, 4)
    codes, s, b = O.quantize(row, 4, "bf16")
    assert s[0] == 1.0 and b[0] == 0.0
    assert codes[:6].tolist() == [0, 15, 0, 2, 2, 4]


def test_constant_group():
    row = np.full(256, 1.375, np.float32)
    row[64:] = RNG.standard_normal(192).astype(np.float32)
    codes, s, b = O.quantize(row, 3, "bf16")
    assert s[0] == 0.0 and b[0] == 1.375
    assert not codes[:64].any()
    assert np.all(O.dequantize(codes, s, b)[:64] == 1.375)


@pytest.mark.parametrize("dist", ["normal", "student_t3", "outliers"])
@pytest.mark.parametrize("bits", [4, 3])
def test_code_range_ends_and_error_bound(bits, dist):
    blocks = seed0_blocks()
    x = W.random_rows(11, (512, 256), "bf16", dist="student_t3" if dist == "student_t3" else "normal")
    x = x.float().numpy()
    if dist == "outliers":
        x[:, [3, 77, 130, 200]] *= 10
    y = O.rotate(x, blocks)
    codes, s, b = O.quantize(y, bits, "bf16")
    top = 2 ** bits - 1
    assert codes.max() <= top
    yg = y.reshape(-1, 4, 64).astype(np.float64)
    cg = codes.reshape(-1, 4, 64)
    s64, b64 = s.astype(np.float64), b.astype(np.float64)
    mn, mx = yg.min(-1), yg.max(-1)
    s32 = ((mx.astype(np.float32) - mn.astype(np.float32)) / np.float32(top)).astype(np.float64)
    # ends: min -> 0 and max -> top whenever |bias - min| < s/2
    ok = np.abs(b64 - mn) < s64 / 2
    amin = np.take_along_axis(cg, yg.argmin(-1)[..., None], -1)[..., 0]
    amax = np.take_along_axis(cg, yg.argmax(-1)[..., None], -1)[..., 0]
    assert np.all(amin[ok] == 0) and np.all(amax[ok] == top)
    # error bound: <= s/2 (up to fp32 rounding of the division) when unclipped,
    # and <= s/2 + |bias - min| + top*|s - s32| in general
    xh = O.dequantize(codes, s, b).reshape(-1, 4, 64)
    err = np.abs(xh - yg)
    raw = (yg - b64[..., None]) / s64[..., None]
    unclipped = (raw > -0.5) & (raw < top + 0.5)
    half = np.broadcast_to((s64 / 2)[..., None], err.shape)
    assert np.all(err[unclipped] <= half[unclipped] * (1 + 2.0 ** -19))
    general = half + (np.abs(b64 - mn) + top * np.abs(s64 - s32))[..., None]
    assert np.all(err <= general * (1 + 2.0 ** -19))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("bits", [4, 3])
def test_quantize_matches_brute(bits, dtype):
    blocks = seed0_blocks()
    x = W.random_rows(12, (6, 256), dtype, dist="student_t3").float().numpy()
    x[0] = 0.5  # constant row
    y = O.rotate(x, blocks)
    codes, s, b = O.quantize(y, bits, dtype)
    for r in range(y.shape[0]):
        bc, bs, bb = brute.quantize_row(y[r].tolist(), bits, dtype)
        assert bc == codes[r].tolist()
        assert bs == s[r].tolist() and bb == b[r].tolist()


# ---------------------------------------------------------------- packing --

def test_packed_widths():
    # _packed_words: dim*bits//32 words; K4 = 32 words = 128 B, V3 = 24 words = 96 B.
    assert O.packed_words(256, 4) == 32 and O.packed_words(256, 4) * 4 == 128
    assert O.packed_words(256, 3) == 24 and O.packed_words(256, 3) * 4 == 96
    for bits in (2, 3, 4, 5, 6, 8):
        assert O.packed_words(256, bits) * 32 == 256 * bits


def _golden_pack():
    rows = []
    with open(os.path.join(GOLDEN, "pack_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, bits, rule, n, *words = line.split()
            rows.append((name, int(bits), int(rule[3:]), [int(w, 16) for w in words]))
    return rows


@pytest.mark.parametrize("case", _golden_pack(), ids=lambda c: c[0])
def test_pack_worked_examples(case):
    name, bits, mod, words = case
    codes = np.arange(256) % mod
    got = O.pack(codes, bits)
    assert got.shape == (O.packed_words(256, bits),)
    assert got[:len(words)].tolist() == words
    assert brute.pack_row(codes.tolist(), bits)[:len(words)] == words


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_pack_matches_bitstring_and_roundtrips(bits):
    codes = RNG.integers(0, 2 ** bits, size=(5, 256))
    words = O.pack(codes, bits)
    for r in range(5):
        assert words[r].tolist() == brute.pack_row(codes[r].tolist(), bits)
        assert brute.unpack_row(words[r].tolist(), bits, 256) == codes[r].tolist()
    np.testing.assert_array_equal(O.unpack(words, bits, 256), codes)


# ------------------------------------------------------------------ cache --

def test_growth_sequence_golden():
    c = O.QuantKVCache()
    with open(os.path.join(GOLDEN, "cache_growth.txt")) as f:
        steps = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for op, n, _, ret, cap, off in steps:
        n, ret, cap, off = int(n), int(ret), int(cap), int(off)
        if op == "append":
            k = W.random_rows([99, n], (1, 1, n, 256), "bf16").float().numpy()
            c.append(k, k, None)
            got = n
        else:
            got = c.trim(n)
        assert (got, c.capacity, c.offset) == (ret, cap, off)
        assert O.required_capacity(0, 0, 1) == 256


def test_trim_and_commit_errors():
    c = O.QuantKVCache()
    k = W.random_rows(5, (1, 1, 10, 256), "bf16").float().numpy()
    c.append(k, k, None)
    with pytest.raises(ValueError):
        c.trim(-1)
    with pytest.raises(ValueError):
        O.commit_verified_prefix(c, 3, 4)
    assert O.commit_verified_prefix(c, 4, 4) == 0 and c.offset == 10
    assert O.commit_verified_prefix(c, 4, 1) == 3 and c.offset == 7
    assert c.trim(100) == 7 and c.offset == 0


def test_append_rows_independent_and_growth_keeps_rows():
    # Appending n rows at once equals n single-row appends, bit for bit
    # (the one-shot vs step-by-step pattern of mtp/kv_cache.py's checkpoint test).
    blocks = seed0_blocks()
    k = W.random_rows(21, (2, 2, 300, 256), "bf16").float().numpy()
    v = W.random_rows(22, (2, 2, 300, 256), "bf16").float().numpy()
    a = O.QuantKVCache()
    a.append(k, v, blocks)
    b = O.QuantKVCache()
    for t in range(300):
        b.append(k[:, :, t:t + 1], v[:, :, t:t + 1], blocks)
    assert a.offset == b.offset == 300
    for name in a.arrays:
        np.testing.assert_array_equal(a.arrays[name][:, :, :300], b.arrays[name][:, :, :300])


# ------------------------------------------------- snapshot / restore --

def _tokens(seed, B, H, n):
    k = W.random_rows([seed, 1], (B, H, n, 256), "bf16").float().numpy()
    v = W.random_rows([seed, 2], (B, H, n, 256), "bf16").float().numpy()
    return k, v


def _fresh(k, v, blocks):
    c = O.QuantKVCache()
    c.append(k, v, blocks)
    return c


def _same_rows(a, b):
    assert a.offset == b.offset
    for name in a.arrays:
        np.testing.assert_array_equal(a.arrays[name][:, :, :a.offset],
                                      b.arrays[name][:, :, :b.offset])


def test_restore_gives_back_the_prefix_of_a_cache_that_never_went_further():
    # A snapshot after t tokens, more tokens, restore: the rows and offset are
    # those of a cache filled with the first t tokens only; appending after the
    # restore equals appending to that cache; the snapshot itself is not
    # changed by what the cache does afterwards.
    blocks = seed0_blocks()
    k, v = _tokens(31, 2, 2, 310)
    t = 300
    c = _fresh(k[:, :, :t], v[:, :, :t], blocks)
    snaps = O.snapshot([c])
    c.append(k[:, :, t:], v[:, :, t:], blocks)
    assert c.offset == 310
    c.trim(20)
    kx, vx = _tokens(32, 2, 2, 6)
    c.append(kx, vx, blocks)  # rewrites rows 290-295, which the snapshot covers
    O.restore([c], snaps)
    ref = _fresh(k[:, :, :t], v[:, :, :t], blocks)
    _same_rows(c, ref)
    # the page's state setter leaves exactly `offset` rows of buffer, so the
    # next append grows from there: 300 + one 256-row step
    assert c.capacity == 300
    c.append(kx[:, :, :5], vx[:, :, :5], blocks)
    assert c.capacity == 556
    ref.append(kx[:, :, :5], vx[:, :, :5], blocks)
    _same_rows(c, ref)
    # restoring twice from one snapshot gives the same state (the restore
    # installs a copy, as the page's _restore does)
    O.restore([c], snaps)
    O.restore([c], snaps)
    _same_rows(c, _fresh(k[:, :, :t], v[:, :, :t], blocks))


def test_snapshot_of_empty_cache_and_meta_state():
    c = O.QuantKVCache()
    snaps = O.snapshot([c])
    assert snaps == [(None, ("64", "4", "3"))]
    k, v = _tokens(33, 1, 1, 10)
    c.append(k, v, None)
    O.restore([c], snaps)
    assert c.arrays is None and c.offset == 0 and c.capacity == 0
    other = O.QuantKVCache(k_bits=8)
    with pytest.raises(ValueError):
        O.restore([other], snaps)


def test_commit_verified_snapshot_cases():
    # Page mtp/kv_cache.py: all accepted -> True, nothing restored;
    # accepted_len outside [1, len(snapshots)] -> False, nothing restored;
    # otherwise the snapshot taken after accepted_len verified tokens.
    blocks = seed0_blocks()
    k, v = _tokens(34, 1, 2, 40)
    c = _fresh(k[:, :, :37], v[:, :, :37], blocks)
    snapshots = []
    for i in range(3):
        c.append(k[:, :, 37 + i:38 + i], v[:, :, 37 + i:38 + i], blocks)
        snapshots.append(O.snapshot([c]))
    assert c.offset == 40
    assert O.commit_verified_snapshot([c], snapshots, 3, verified_len=3) is True
    assert c.offset == 40
    assert O.commit_verified_snapshot([c], snapshots, 0) is False and c.offset == 40
    assert O.commit_verified_snapshot([c], snapshots, 4) is False and c.offset == 40
    assert O.commit_verified_snapshot([c], snapshots, 2, verified_len=3) is True
    _same_rows(c, _fresh(k[:, :, :39], v[:, :, :39], blocks))


# -------------------------------------------------------------- attention --

def _small_cache(seed, B, Hkv, T, dtype="bf16", blocks=None):
    c = O.QuantKVCache(dtype=dtype)
    k = W.random_rows([seed, 1], (B, Hkv, T, 256), dtype).float().numpy()
    v = W.random_rows([seed, 2], (B, Hkv, T, 256), dtype).float().numpy()
    c.append(k, v, blocks)
    return c


@pytest.mark.parametrize("rot", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_matches_brute(rot, causal):
    blocks = seed0_blocks() if rot else None
    B, Hq, Hkv, T, L = 1, 4, 2, 37, 3
    c = _small_cache(31, B, Hkv, T, blocks=blocks)
    q = W.random_rows(32, (B, Hq, L, 256), "bf16").float().numpy()
    out = O.attention(q, c, 1 / 16, causal, blocks)
    for h in range(Hq):
        kh, vh = c.dequant_kv(0, h // 2)
        for i in range(L):
            n = T - L + i + 1 if causal else T
            ref = brute.attention_row(q[0, h, i].tolist(), kh.tolist(), vh.tolist(), n, 1 / 16,
                                      None if blocks is None else blocks.tolist())
            np.testing.assert_allclose(out[0, h, i], ref, rtol=0, atol=1e-6)


def test_attention_matches_torch_sdpa_without_rotation():
    # With no rotation the path is plain softmax(q k^T * scale) v over the
    # dequantised cache: compare with torch's SDPA in fp64 on the CPU.
    B, Hq, Hkv, T, L = 2, 8, 2, 300, 4
    c = _small_cache(41, B, Hkv, T)
    q = W.random_rows(42, (B, Hq, L, 256), "bf16").float().numpy()
    out = O.attention(q, c, 1 / 16, True, None)
    K = np.stack([np.stack([c.dequant_kv(b, h)[0] for h in range(Hkv)]) for b in range(B)])
    V = np.stack([np.stack([c.dequant_kv(b, h)[1] for h in range(Hkv)]) for b in range(B)])
    K = np.repeat(K, Hq // Hkv, axis=1)
    V = np.repeat(V, Hq // Hkv, axis=1)
    mask = torch.arange(T)[None, :] <= (T - L + torch.arange(L))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q.astype(np.float64)), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=mask, scale=1 / 16)
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-6)


def test_single_key_and_identical_keys():
    blocks = seed0_blocks()
    c = _small_cache(51, 1, 1, 1, blocks=blocks)
    q = W.random_rows(52, (1, 1, 1, 256), "bf16").float().numpy()
    out = O.attention(q, c, 1 / 16, True, blocks)
    _, v0 = c.dequant_kv(0, 0)
    np.testing.assert_allclose(out[0, 0, 0], O.inverse_rotate(v0[0].astype(np.float32), blocks),
                               atol=1e-6)
    # identical keys -> uniform weights -> mean of the values
    c2 = O.QuantKVCache()
    k = np.repeat(W.random_rows(53, (1, 1, 1, 256), "bf16").float().numpy(), 50, axis=2)
    v = W.random_rows(54, (1, 1, 50, 256), "bf16").float().numpy()
    c2.append(k, v, blocks)
    out2 = O.attention(q, c2, 1 / 16, False, blocks)
    _, vh = c2.dequant_kv(0, 0)
    np.testing.assert_allclose(out2[0, 0, 0],
                               O.inverse_rotate(vh.mean(0).astype(np.float32), blocks), atol=1e-6)


def test_array_masks():
    # asym_quantized_sdpa's array masks: a boolean mask of the causal pattern
    # is the causal mask (the page builds its "causal" string mask exactly so:
    # q index >= k index); an all-true mask or an additive zero mask changes
    # nothing; an additive constant shifts every score alike (softmax
    # invariance); an additive -inf drops a key exactly as a false boolean.
    blocks = seed0_blocks()
    B, Hkv, Hq, T, L = 1, 2, 4, 70, 3
    c = _small_cache(61, B, Hkv, T, blocks=blocks)
    q = W.random_rows(62, (B, Hq, L, 256), "bf16").float().numpy()
    base_c = O.attention(q, c, 1 / 16, True, blocks)
    base_n = O.attention(q, c, 1 / 16, False, blocks)
    qi = np.arange(T - L, T)[:, None]
    causal = qi >= np.arange(T)[None]
    np.testing.assert_array_equal(O.attention(q, c, 1 / 16, False, blocks, mask=causal), base_c)
    np.testing.assert_array_equal(
        O.attention(q, c, 1 / 16, False, blocks, mask=np.ones((L, T), bool)), base_n)
    np.testing.assert_array_equal(
        O.attention(q, c, 1 / 16, False, blocks, mask=np.zeros((1, 1, L, T))), base_n)
    np.testing.assert_allclose(
        O.attention(q, c, 1 / 16, False, blocks, mask=np.full((L, T), -7.5)), base_n, atol=1e-6)
    rng = np.random.default_rng(63)
    keep = rng.random((B, Hq, L, T)) < 0.6
    keep[..., 0] = True
    add = np.where(keep, 0.0, -np.inf)
    np.testing.assert_array_equal(O.attention(q, c, 1 / 16, False, blocks, mask=keep),
                                  O.attention(q, c, 1 / 16, False, blocks, mask=add))
    # one kept key: the output is that key's value; no kept key: the page's
    # minimum fill makes every score equal, so all keys weigh alike
    one = np.zeros((L, T), bool)
    one[:, 17] = True
    _, vh = c.dequant_kv(0, 0)
    out1 = O.attention(q, c, 1 / 16, False, blocks, mask=one)
    np.testing.assert_allclose(out1[0, 0, 1], O.inverse_rotate(vh[17].astype(np.float32), blocks),
                               atol=1e-6)
    none = np.zeros((L, T), bool)
    out0 = O.attention(q, c, 1 / 16, False, blocks, mask=none)
    np.testing.assert_allclose(out0[0, 1, 2], O.inverse_rotate(vh.mean(0).astype(np.float32),
                                                                 blocks), atol=1e-6)
    # brute force on a masked row
    kh1, vh1 = c.dequant_kv(0, 1)  # q head 3 reads kv head 1
    kept = np.flatnonzero(keep[0, 3, 1])
    ref = brute.attention_row(q[0, 3, 1], kh1[kept], vh1[kept], len(kept), 1 / 16, blocks)
    got = O.attention(q, c, 1 / 16, False, blocks, mask=keep)[0, 3, 1]
    np.testing.assert_allclose(got, ref, atol=2e-6)


def test_tile_and_commit_tree_row():
    # tile_caches: every batch row of the tiled cache is the batch-1 cache;
    # commit_tree_row: trim the rejected suffix and keep the winning row, equal
    # to a cache that saw only that path's accepted tokens.
    blocks = seed0_blocks()
    k, v = _tokens(64, 1, 2, 50)
    c = _fresh(k, v, blocks)
    O.tile_cache(c, 3)
    assert c.offset == 50 and c.arrays["kw"].shape[0] == 3 and c.capacity == 50
    ref = _fresh(k, v, blocks)
    for b in range(3):
        for name in c.arrays:
            np.testing.assert_array_equal(c.arrays[name][b:b + 1], ref.arrays[name][:, :, :50])
    paths = [_tokens(65 + p, 1, 2, 4) for p in range(3)]
    kp = np.concatenate([pk for pk, _ in paths], 0)
    vp = np.concatenate([pv for _, pv in paths], 0)
    c.append(kp, vp, blocks)
    assert O.commit_tree_row([c], 4, 2, 1) is True
    win = _fresh(np.concatenate([k, paths[1][0][:, :, :2]], 2),
                 np.concatenate([v, paths[1][1][:, :, :2]], 2), blocks)
    _same_rows(c, win)
    assert c.arrays["kw"].shape[0] == 1
    with pytest.raises(ValueError):
        O.commit_tree_row([c], 2, 3, 0)
    with pytest.raises(ValueError):
        O.tile_cache(_fresh(np.concatenate([k, k]), np.concatenate([v, v]), blocks), 2)


def test_causal_row_equals_shorter_decode():
    # asym_quantized_sdpa's causal mask at the offset: row i of an L-block
    # sees keys t <= T - L + i, i.e. equals an L = 1 decode over T - L + i + 1 keys.
    blocks = seed0_blocks()
    T, L = 90, 4
    c = _small_cache(61, 1, 2, T, blocks=blocks)
    q = W.random_rows(62, (1, 4, L, 256), "bf16").float().numpy()
    out = O.attention(q, c, 1 / 16, True, blocks)
    for i in range(L):
        c.offset = T - L + i + 1
        one = O.attention(q[:, :, i:i + 1], c, 1 / 16, True, blocks)
        np.testing.assert_array_equal(one[:, :, 0], out[:, :, i])
    c.offset = T


def test_rotation_cancels_in_scores_and_output():
    # With the rotation, attention over the rotated cache followed by the
    # inverse rotation equals attention of the unrotated q over K_hat M^T, V_hat M^T.
    blocks = seed0_blocks()
    M = O.dense_rotation(blocks)
    T = 64
    c = _small_cache(71, 1, 1, T, blocks=blocks)
    q = W.random_rows(72, (1, 1, 1, 256), "bf16").float().numpy()
    out = O.attention(q, c, 1 / 16, True, blocks)[0, 0, 0]
    kh, vh = c.dequant_kv(0, 0)
    s = (kh @ M.T) @ q[0, 0, 0].astype(np.float64) / 16
    p = np.exp(s - s.max())
    ref = (p / p.sum()) @ (vh @ M.T)
    np.testing.assert_allclose(out, ref, atol=1e-6)


def test_gqa_head_mapping():
    # q head h reads kv head h // (Hq/Hkv): give each kv head constant values.
    Hq, Hkv, T = 8, 4, 10
    c = O.QuantKVCache()
    k = W.random_rows(81, (1, Hkv, T, 256), "bf16").float().numpy()
    v = np.zeros((1, Hkv, T, 256), np.float32)
    for h in range(Hkv):
        v[0, h] = float(h + 1)
    c.append(k, v, None)
    q = W.random_rows(82, (1, Hq, 1, 256), "bf16").float().numpy()
    out = O.attention(q, c, 1 / 16, True, None)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h, 0], float(h // 2 + 1), atol=1e-6)


def test_attention_shape_errors():
    c = _small_cache(91, 1, 2, 4)
    with pytest.raises(ValueError):
        O.attention(np.zeros((1, 3, 1, 256), np.float32), c, 1 / 16, True, None)
    with pytest.raises(ValueError):
        O.attention(np.zeros((1, 2, 5, 256), np.float32), c, 1 / 16, True, None)

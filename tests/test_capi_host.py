"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-only entry points agree with the oracle; device entry points reject
bad arguments before any device work (no GPU call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import workloads as W
from oracle import rbq_oracle as O

rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "rbq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rbq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = declared_symbols()
    for name in ("rbq_rotation_build", "rbq_kv_quant_append", "rbq_kv_trim",
                 "rbq_quant_attn_decode"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(capi.LIB_PATH)
    missing = [s for s in declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing


@pytest.mark.parametrize("seed", [0, 1, 12345])
def test_rotation_build_bit_exact_vs_oracle(seed):
    draws = W.rotation_draws(seed, 256)
    got = capi.rbq_rotation_build(draws)
    np.testing.assert_array_equal(got, O.rotation_blocks(draws))


def test_package_draws_match_the_input_generator():
    # The package's seed -> draws step and the shared generator take the same
    # numbers from numpy's default_rng in the same order.
    np.testing.assert_array_equal(rbq.quaternion_draws(0, 256), W.rotation_draws(0, 256))


def test_rotation_build_other_head_dims_and_errors():
    for D in (4, 64, 128):
        draws = W.rotation_draws(3, D)
        np.testing.assert_array_equal(capi.rbq_rotation_build(draws), O.rotation_blocks(draws))
    bad = np.zeros((2, 2, 4), np.float32)
    bad[0] = 1.0
    with pytest.raises(capi.RbqError):
        capi.rbq_rotation_build(bad)  # block 1 has a zero-norm draw
    assert capi.library().rbq_rotation_build(None, 256, None) == capi.RBQ_EINVAL
    d = np.ones((1, 2, 4), np.float32)
    out = np.empty((1, 4, 4), np.float32)
    assert capi.library().rbq_rotation_build(d.ctypes.data, 6, out.ctypes.data) == capi.RBQ_EINVAL


@pytest.mark.parametrize("D", [64, 128, 256])
def test_rotation_build_two_sided_bit_exact_vs_oracle(D):
    draws = W.rotation_draws(7, D)
    got = capi.rbq_rotation_build_mode(draws, capi.RBQ_ROT_TWO_SIDED)
    np.testing.assert_array_equal(got, O.rotation_blocks(draws, mode="two_sided"))
    np.testing.assert_array_equal(capi.rbq_rotation_build_mode(draws, capi.RBQ_ROT_PRINTED),
                                  capi.rbq_rotation_build(draws))
    d = np.ascontiguousarray(draws)
    out = np.empty((D // 4, 4, 4), np.float32)
    assert capi.library().rbq_rotation_build_mode(d.ctypes.data, D, 2, out.ctypes.data) == \
        capi.RBQ_EINVAL


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mode", ["printed", "two_sided"])
def test_rotation_round_bit_exact_vs_oracle(dtype, mode):
    # the page's own rotation precision: blocks rounded to the cache dtype by
    # the library, against the oracle's rounding of the oracle's blocks
    code = capi.RBQ_BF16 if dtype == "bf16" else capi.RBQ_F16
    for D, seed in ((256, 0), (128, 5), (64, 9)):
        draws = W.rotation_draws(seed, D)
        cmode = capi.RBQ_ROT_TWO_SIDED if mode == "two_sided" else capi.RBQ_ROT_PRINTED
        got = capi.rbq_rotation_round(capi.rbq_rotation_build_mode(draws, cmode), code)
        want = O.round_to_dtype(O.rotation_blocks(draws, mode=mode), dtype)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rotation_round_ties_subnormals_overflow(dtype):
    # the rounding on its own, over values that are not rotation entries:
    # exact ties, fp16 subnormal halves, values that round up to the next
    # power of two and past the largest finite value
    code = capi.RBQ_BF16 if dtype == "bf16" else capi.RBQ_F16
    rng = np.random.default_rng(31)
    x = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000),
        np.float32(1.0) + np.float32(2.0 ** -11) * np.arange(-8, 9),   # fp16 ties around 1
        np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(-8, 9),    # bf16 ties around 1
        np.float32(2.0 ** -24) * np.arange(0, 40) / 4,                  # fp16 subnormal ties
        np.array([65504.0, 65519.0, 65520.0, 65536.0, 3.3e38, -65520.0, 2.0 ** -25,
                  3.0 * 2.0 ** -26, 0.0, -0.0]),
    ]).astype(np.float32)
    x = x[: (x.size // 64) * 64].reshape(-1, 4, 4)
    with np.errstate(over="ignore"):
        want = O.round_to_dtype(x, dtype)
    got = capi.rbq_rotation_round(x, code)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    bad = np.ones((1, 4, 4), np.float32)
    bad[0, 1, 2] = np.inf
    with pytest.raises(capi.RbqError):
        capi.rbq_rotation_round(bad, code)
    assert capi.library().rbq_rotation_round(bad.ctypes.data, 4, 7) == capi.RBQ_EUNSUPPORTED
    assert capi.library().rbq_rotation_round(None, 4, code) == capi.RBQ_EINVAL


def test_required_capacity_matches_oracle():
    for cap in (0, 256, 512, 8192, 10240, 10496):
        for off in sorted({0, 1, cap // 2, max(cap - 1, 0), cap, 255, 257}):
            if off > cap:
                continue
            for n in (0, 1, 2, 255, 256, 257, 2048, 4096 + 3):
                if cap == 0 and off != 0:
                    continue
                assert capi.rbq_kv_required_capacity(cap, off, n) == \
                    O.required_capacity(cap, off, n), (cap, off, n)
    for args in ((0, 0, -1), (10, 11, 1), (-1, 0, 0)):
        with pytest.raises(capi.RbqError):
            capi.rbq_kv_required_capacity(*args)


def _host_desc(B=1, H=1, cap=0, off=0, dtype=capi.RBQ_BF16, **kw):
    d = capi.rbq_kv_cache(B=B, H_kv=H, head_dim=256, group_size=64, k_bits=4, v_bits=3,
                          dtype=dtype, flags=0, capacity=cap, offset=off)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_growth_golden_through_the_library():
    # Capacity/offset sequence of the append+verify workload (tests/golden/cache_growth.txt),
    # replayed with the library's capacity rule and trim.
    d = _host_desc()
    with open(os.path.join(GOLDEN, "cache_growth.txt")) as f:
        steps = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for op, n, _, ret, cap, off in steps:
        n, ret, cap, off = int(n), int(ret), int(cap), int(off)
        if op == "append":
            d.capacity = capi.rbq_kv_required_capacity(d.capacity, d.offset, n)
            d.offset += n
            got = n
        else:
            got = capi.rbq_kv_trim(d, n)
        assert (got, d.capacity, d.offset) == (ret, cap, off)


def test_trim_and_commit_semantics():
    d = _host_desc(cap=256, off=10)
    with pytest.raises(capi.RbqError):
        capi.rbq_kv_trim(d, -1)
    with pytest.raises(capi.RbqError):
        capi.rbq_kv_commit_verified(d, 3, 4)
    assert capi.rbq_kv_commit_verified(d, 4, 4) == 0 and d.offset == 10
    assert capi.rbq_kv_commit_verified(d, 4, 1) == 3 and d.offset == 7
    assert capi.rbq_kv_trim(d, 100) == 7 and d.offset == 0


def test_device_entry_points_validate_before_any_device_work():
    lib = capi.library()
    fake = 0x1000  # never dereferenced: every call below fails validation first
    ptrs = dict(k_words=fake, k_scales=fake, k_biases=fake, v_words=fake, v_scales=fake,
                v_biases=fake)
    d = _host_desc(B=1, H=2, cap=256, off=100, **ptrs)
    by = ctypes.byref
    # append: capacity exceeded, negative n, null inputs
    assert lib.rbq_kv_quant_append(by(d), fake, fake, 157, None, None) == capi.RBQ_ECAPACITY
    assert d.offset == 100
    assert lib.rbq_kv_quant_append(by(d), fake, fake, -1, None, None) == capi.RBQ_EINVAL
    assert lib.rbq_kv_quant_append(by(d), None, fake, 1, None, None) == capi.RBQ_EINVAL
    assert lib.rbq_kv_quant_append(by(d), fake, fake, 0, None, None) == capi.RBQ_OK
    # unsupported configurations
    for field, val in (("head_dim", 96), ("head_dim", 512), ("group_size", 16),
                       ("group_size", 256), ("k_bits", 7), ("k_bits", 1), ("v_bits", 16),
                       ("dtype", 7)):
        e = _host_desc(B=1, H=2, cap=256, off=100, **ptrs)
        setattr(e, field, val)
        assert lib.rbq_kv_quant_append(by(e), fake, fake, 1, None, None) == \
            capi.RBQ_EUNSUPPORTED, (field, val)
    e = _host_desc(B=1, H=2, cap=256, off=100, head_dim=64, group_size=128, **ptrs)
    assert lib.rbq_kv_quant_append(by(e), fake, fake, 1, None, None) == capi.RBQ_EUNSUPPORTED
    # supported variants pass validation (here they stop at the capacity check)
    for hd, gs, kb, vb in ((64, 32, 2, 8), (128, 64, 5, 6), (256, 128, 8, 2), (64, 64, 3, 3)):
        e = _host_desc(B=1, H=2, cap=256, off=100, head_dim=hd, group_size=gs, k_bits=kb,
                       v_bits=vb, **ptrs)
        assert lib.rbq_kv_quant_append(by(e), fake, fake, 157, None, None) == capi.RBQ_ECAPACITY
    # misaligned arrays (the kernels move words in 16-byte, scales in 4-byte pieces)
    for field, val in (("k_words", fake + 4), ("v_words", fake + 8), ("k_scales", fake + 2),
                       ("v_biases", fake + 2)):
        e = _host_desc(B=1, H=2, cap=256, off=100, **ptrs)
        setattr(e, field, val)
        assert lib.rbq_kv_quant_append(by(e), fake, fake, 1, None, None) == capi.RBQ_EINVAL, field
    e = _host_desc(B=1, H=2, cap=256, off=100, **ptrs)
    e.flags = 2
    assert lib.rbq_kv_quant_append(by(e), fake, fake, 1, None, None) == capi.RBQ_EINVAL
    e.flags = capi.RBQ_FLAG_ROUND_ROTATED
    assert lib.rbq_kv_quant_append(by(e), fake, fake, 157, None, None) == capi.RBQ_ECAPACITY
    e = _host_desc(B=1, H=2, cap=256, off=300, **ptrs)
    assert lib.rbq_kv_quant_append(by(e), fake, fake, 1, None, None) == capi.RBQ_EINVAL
    # attention: H_q % H_kv, L range, splits < 0, null q/out, workspace
    dec = lib.rbq_quant_attn_decode
    assert dec(by(d), fake, 3, 1, 0.0625, 1, None, fake, 0, None, 0, None) == capi.RBQ_EINVAL
    assert dec(by(d), fake, 4, 0, 0.0625, 1, None, fake, 0, None, 0, None) == capi.RBQ_ERANGE
    assert dec(by(d), fake, 4, 101, 0.0625, 1, None, fake, 0, None, 0, None) == capi.RBQ_ERANGE
    assert dec(by(d), fake, 4, 1, 0.0625, 1, None, fake, -2, None, 0, None) == capi.RBQ_EINVAL
    assert dec(by(d), None, 4, 1, 0.0625, 1, None, fake, 0, None, 0, None) == capi.RBQ_EINVAL
    # misaligned q / out / rotation blocks / workspace
    assert dec(by(d), fake + 4, 4, 1, 0.0625, 1, None, fake, 0, None, 0, None) == capi.RBQ_EINVAL
    assert dec(by(d), fake, 4, 1, 0.0625, 1, None, fake + 8, 0, None, 0, None) == capi.RBQ_EINVAL
    assert dec(by(d), fake, 4, 1, 0.0625, 1, fake + 4, fake, 0, None, 0, None) == capi.RBQ_EINVAL
    assert dec(by(d), fake, 4, 1, 0.0625, 1, None, fake, 0, fake + 4, 1 << 30, None) == capi.RBQ_EINVAL
    need = lib.rbq_quant_attn_workspace_bytes(by(d), 4, 1, 8)
    assert need > 0
    assert dec(by(d), fake, 4, 1, 0.0625, 1, None, fake, 8, None, 0, None) == capi.RBQ_EWORKSPACE
    assert dec(by(d), fake, 4, 1, 0.0625, 1, None, fake, 8, fake, need - 1, None) == \
        capi.RBQ_EWORKSPACE
    assert lib.rbq_quant_attn_splits(by(d), 4, 1) >= 1
    assert lib.rbq_quant_attn_splits(by(d), 3, 1) == capi.RBQ_EINVAL
    # append + attention in one call: every argument of both steps is checked
    # before a launch, and an error leaves the offset where it was
    fused = lib.rbq_kv_append_attn_decode
    off0 = d.offset
    args = lambda **kw: dict(dict(k=fake, v=fake, n=1, q=fake, H_q=4, L=1, rot=None, out=fake,
                                  splits=0, ws=fake, nb=1 << 30), **kw)

    def call(**kw):
        a = args(**kw)
        return fused(by(d), a["k"], a["v"], a["n"], a["q"], a["H_q"], a["L"], 0.0625, 1,
                     a["rot"], a["out"], a["splits"], a["ws"], a["nb"], None)

    assert call(n=-1) == capi.RBQ_EINVAL
    assert call(k=None) == capi.RBQ_EINVAL
    assert call(v=None) == capi.RBQ_EINVAL
    assert call(n=157) == capi.RBQ_ECAPACITY
    assert call(H_q=3) == capi.RBQ_EINVAL
    assert call(L=0) == capi.RBQ_ERANGE
    assert call(n=2, L=103) == capi.RBQ_ERANGE  # the block may reach the appended rows only
    assert call(q=None) == capi.RBQ_EINVAL
    assert call(q=fake + 4) == capi.RBQ_EINVAL
    assert call(out=fake + 8) == capi.RBQ_EINVAL
    assert call(rot=fake + 4) == capi.RBQ_EINVAL
    assert call(splits=-1) == capi.RBQ_EINVAL
    assert call(splits=8, ws=None, nb=0) == capi.RBQ_EWORKSPACE
    after = _host_desc(B=1, H=2, cap=256, off=off0 + 1, **ptrs)
    need1 = lib.rbq_quant_attn_workspace_bytes(by(after), 4, 1, 8)
    assert need1 > 0
    assert call(splits=8, nb=need1 - 1) == capi.RBQ_EWORKSPACE
    assert d.offset == off0
    # grow: mismatched descriptors
    g = _host_desc(B=2, H=2, cap=512, off=0, **ptrs)
    assert lib.rbq_kv_grow(by(d), by(g), None) == capi.RBQ_EINVAL
    # prefix copy: mismatched descriptors, destination too small, overlap
    assert lib.rbq_kv_copy_prefix(by(d), by(g), None) == capi.RBQ_EINVAL
    small = _host_desc(B=1, H=2, cap=99, off=0, k_words=0x9000000, k_scales=0xA000000,
                       k_biases=0xB000000, v_words=0xC000000, v_scales=0xD000000,
                       v_biases=0xE000000)
    assert lib.rbq_kv_copy_prefix(by(d), by(small), None) == capi.RBQ_ECAPACITY
    assert small.offset == 0
    same = _host_desc(B=1, H=2, cap=256, off=0, **ptrs)
    assert lib.rbq_kv_copy_prefix(by(d), by(same), None) == capi.RBQ_EINVAL
    empty = _host_desc(B=1, H=2, cap=256, off=0, **ptrs)
    tgt = _host_desc(B=1, H=2, cap=0, off=0)
    tgt.offset = 0
    assert lib.rbq_kv_copy_prefix(by(empty), by(tgt), None) == capi.RBQ_OK and tgt.offset == 0
    # batch gather: source entries outside the source batch
    two = _host_desc(B=2, H=2, cap=256, off=50, k_words=0x9000000, k_scales=0xA000000,
                     k_biases=0xB000000, v_words=0xC000000, v_scales=0xD000000,
                     v_biases=0xE000000)
    assert lib.rbq_kv_copy_batch(by(d), 1, 0, by(two), None) == capi.RBQ_EINVAL
    assert lib.rbq_kv_copy_batch(by(d), 0, 1, by(two), None) == capi.RBQ_EINVAL
    assert lib.rbq_kv_copy_batch(by(d), -1, 1, by(two), None) == capi.RBQ_EINVAL
    # masked attention: mask type / strides validated before any device work
    mdec = lib.rbq_quant_attn_decode_mask
    assert mdec(by(d), fake, 4, 1, 0.0625, 1, fake, 7, 0, 0, 0, None, fake, 0, None, 0,
                None) == capi.RBQ_EINVAL
    assert mdec(by(d), fake, 4, 1, 0.0625, 1, fake, capi.RBQ_MASK_BOOL, 0, -5, 0, None, fake, 0,
                None, 0, None) == capi.RBQ_EINVAL
    assert mdec(by(d), fake, 4, 1, 0.0625, 1, fake, capi.RBQ_MASK_ADD_F32, 0, 1 << 28, 0, None,
                fake, 0, None, 0, None) == capi.RBQ_EUNSUPPORTED  # 3 heads x 2^28 x 4 B


def test_automatic_split_counts():
    """The automatic plan of the default configuration: about one workgroup per
    compute unit, whole 256-key rounds per split with one block of 8 query rows
    per kv head; with several row blocks a multiple of 8 splits (whole 32-key
    tiles), so that the row blocks of one (b, kv head, split) share an XCD."""
    lib = capi.library()
    fake = 0x1000
    ptrs = dict(k_words=fake, k_scales=fake, k_biases=fake, v_words=fake, v_scales=fake,
                v_biases=fake)
    by = ctypes.byref
    cases = [  # B, T, H_q, L, splits
        (8, 32768, 16, 1, 16),    # 16 (b, kv head) units, 2048 keys each
        (1, 262144, 16, 1, 128),
        (1, 4096, 16, 1, 16),
        (1, 256, 2, 1, 1),        # one round of 8 tiles: one split
        (4, 10244, 16, 4, 8),     # 4 row blocks per kv head: 8 splits of 41 tiles
        (4, 10242, 16, 2, 16),    # 2 row blocks: 16 splits of 21 tiles
        (8, 1000, 16, 2, 4),      # 8 splits would leave waves without a tile: rounds
        (1, 10240, 16, 2048, 1),  # 4096 row blocks fill the chip alone
    ]
    for B, T, hq, L, want in cases:
        d = _host_desc(B=B, H=2, cap=T + 256, off=T, **ptrs)
        assert lib.rbq_quant_attn_splits(by(d), hq, L) == want, (B, T, hq, L)
        ws = lib.rbq_quant_attn_workspace_bytes(by(d), hq, L, 0)
        rb = (hq // 2 * L + 7) // 8
        assert ws == (0 if want == 1 else B * 2 * rb * want * (16 + 8 * 256) * 4)


def test_launch_sizes_are_bounded():
    """Calls whose kernels would need more than 2^32 - 1 work-items along x in
    one launch are refused before any device work."""
    lib = capi.library()
    fake = 0x1000
    ptrs = dict(k_words=fake, k_scales=fake, k_biases=fake, v_words=fake, v_scales=fake,
                v_biases=fake)
    by = ctypes.byref
    dec = lib.rbq_quant_attn_decode
    # default configuration, 2^21 (b, kv head) units: with key splits the
    # merge kernel would need 2^21 x 8 x 512 work-items
    d = _host_desc(B=1 << 20, H=2, cap=4096, off=4096, **ptrs)
    assert dec(by(d), fake, 4, 1, 0.0625, 1, None, fake, 2, fake, 1 << 62, None) == \
        capi.RBQ_EUNSUPPORTED
    assert lib.rbq_quant_attn_splits(by(d), 4, 1) == 1  # one split: no merge, planned
    # head_dim 128 K4/V4: 2^21 units, one 256-thread merge workgroup per row
    # (16 per unit)
    e = _host_desc(B=1 << 20, H=2, cap=4096, off=4096, head_dim=128, group_size=64, k_bits=4,
                   v_bits=4, **ptrs)
    assert dec(by(e), fake, 16, 1, 0.0884, 1, None, fake, 2, fake, 1 << 62, None) == \
        capi.RBQ_EUNSUPPORTED


def test_prepared_step_checks_its_arguments():
    import torch
    d = _host_desc(B=1, H=2, cap=256, off=100, k_words=0x1000, k_scales=0x1000, k_biases=0x1000,
                   v_words=0x1000, v_scales=0x1000, v_biases=0x1000)
    k = torch.zeros(1, 2, 1, 256, dtype=torch.bfloat16)
    q = torch.zeros(1, 4, 1, 256, dtype=torch.bfloat16)
    out = torch.zeros(1, 4, 1, 256, dtype=torch.float32)
    with pytest.raises(ValueError):  # host tensors
        capi.prepare_append_attn_decode(d, k, k, q, 0.0625, True, None, out)
    with pytest.raises(ValueError):  # k / v shapes differ
        capi.prepare_append_attn_decode(d, k, k[:, :1], q, 0.0625, True, None, out)
    with pytest.raises(ValueError):  # out shape
        capi.prepare_append_attn_decode(d, k, k, q, 0.0625, True, None, out[:, :2])


def test_status_strings():
    lib = capi.library()
    for st in range(0, -7, -1):
        assert lib.rbq_status_string(st).decode() not in ("", "unknown status")
    assert lib.rbq_status_string(-99).decode() == "unknown status"


def test_prefill_plan_selection():
    """Which plan a call gets: from 96 query rows per kv head over a bf16 or
    fp16 cache with 4-bit K in groups of 64 or 128 the prefill kernel's (128-row
    blocks, split records of 8 rows at head_dim 256, 128 and 64); below that
    the dedicated kernel's (8-row blocks, a multiple of 8 splits with several
    row blocks); other widths the tile kernel's."""
    lib = capi.library()
    fake = 0x1000
    ptrs = dict(k_words=fake, k_scales=fake, k_biases=fake, v_words=fake, v_scales=fake,
                v_biases=fake)
    by = ctypes.byref
    rec = (16 + 8 * 256) * 4
    # default layout, bf16, 96 rows per kv head (16 q heads / 2, L = 12): two
    # 128-row blocks, 128 splits capped at one 256-key round each (40)
    d = _host_desc(B=1, H=2, cap=10496, off=10240, **ptrs)
    assert lib.rbq_quant_attn_splits(by(d), 16, 12) == 40
    assert lib.rbq_quant_attn_workspace_bytes(by(d), 16, 12, 0) == 2 * 12 * 40 * rec
    # 88 rows: the dedicated kernel, 11 row blocks -> 16 splits
    assert lib.rbq_quant_attn_splits(by(d), 16, 11) == 16
    # the same 96 rows over an fp16 cache: the prefill kernel too; 88 rows:
    # the dedicated kernel
    d16 = _host_desc(B=1, H=2, cap=10496, off=10240, dtype=capi.RBQ_F16, **ptrs)
    assert lib.rbq_quant_attn_splits(by(d16), 16, 12) == 40
    assert lib.rbq_quant_attn_workspace_bytes(by(d16), 16, 12, 0) == 2 * 12 * 40 * rec
    assert lib.rbq_quant_attn_splits(by(d16), 16, 11) == 16
    # head_dim 128, K4/V4, group 64, bf16: 2048-token chunk of 16 q heads / 2
    # (256 blocks of 128 rows): the prefill kernel, one split, no workspace
    d128 = _host_desc(B=1, H=2, cap=10496, off=10240, **ptrs)
    d128.head_dim, d128.v_bits = 128, 4
    assert lib.rbq_quant_attn_splits(by(d128), 16, 2048) == 1
    assert lib.rbq_quant_attn_workspace_bytes(by(d128), 16, 2048, 0) == 0
    # 256 rows per kv head (2 blocks of 128): the prefill kernel with key
    # splits (40, one 256-key round each) and records of head_dim 128; an
    # explicit single split: no records
    rec128 = (16 + 8 * 128) * 4
    assert lib.rbq_quant_attn_splits(by(d128), 16, 32) == 40
    assert lib.rbq_quant_attn_workspace_bytes(by(d128), 16, 32, 0) == 2 * 32 * 40 * rec128
    assert lib.rbq_quant_attn_workspace_bytes(by(d128), 16, 32, 1) == 0
    # groups of 128 dims: the prefill kernel from 96 rows (same splits and
    # records as groups of 64), the tile kernel below (the dedicated kernel
    # takes groups of 64 only); groups of 32: the tile kernel at any row count
    g128 = _host_desc(B=1, H=2, cap=10496, off=10240, **ptrs)
    g128.group_size = 128
    assert lib.rbq_quant_attn_splits(by(g128), 16, 12) == 40
    assert lib.rbq_quant_attn_workspace_bytes(by(g128), 16, 12, 0) == 2 * 12 * 40 * rec
    assert lib.rbq_quant_attn_splits(by(g128), 16, 11) not in (16, 40)
    assert lib.rbq_quant_attn_splits(by(g128), 16, 2048) == 1
    g32 = _host_desc(B=1, H=2, cap=10496, off=10240, **ptrs)
    g32.group_size = 32
    assert lib.rbq_quant_attn_splits(by(g32), 16, 12) == lib.rbq_quant_attn_splits(by(g128), 16, 11)
    # a group of 128 over a head of 64: a layout not built
    g128.head_dim = 64
    assert lib.rbq_quant_attn_splits(by(g128), 16, 12) == capi.RBQ_EUNSUPPORTED
    # 5-bit K codes: the tile kernel
    d5 = _host_desc(B=1, H=2, cap=10496, off=10240, **ptrs)
    d5.head_dim, d5.k_bits, d5.v_bits = 128, 5, 4
    assert lib.rbq_quant_attn_workspace_bytes(by(d5), 16, 2048, 1) == 0
    assert lib.rbq_quant_attn_splits(by(d5), 16, 2048) >= 1

"""GPU parity of the tile kernel's register-staged shape against the oracle.

Up to 8 query rows per kv head with 4-bit K codes and 2-, 3- or 4-bit V
codes at head_dim 64 and 128 run single-wave workgroups that load each
tile's packed words and scale / bias halves into registers two tiles ahead
and pair the hi and lo parts of the query rows in one matrix operand.
Covered here: both head dims, every group count (1, 2 and 4 groups per row),
the three V widths, both dtypes, both rotations and the page's rotation
precision; 4 and 8 rows per kv head (GQA rows and causal verify rows), a
ragged last tile, one split (many tiles per workgroup: both register sets
and the odd last tile), automatic and explicit splits; an additive mask and
a boolean mask with rows that keep no key.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O

pytestmark = pytest.mark.gpu

ATOL = 2e-3
rbq = pytest.importorskip("rotated_bit_quantized_amd")

# (head_dim, group, k_bits, v_bits, dtype, two-sided rotation, rotation in the dtype)
VARS = [
    (64, 32, 4, 4, "f16", False, False),
    (64, 64, 4, 4, "bf16", True, False),
    (128, 128, 4, 4, "f16", False, True),
    (128, 32, 4, 4, "bf16", True, False),
    (128, 64, 4, 4, "bf16", True, True),
    (128, 64, 4, 3, "bf16", False, False),
    (64, 32, 4, 2, "f16", True, False),
    (128, 32, 4, 3, "f16", False, True),
]
# (B, H_q, H_kv, L): rows per kv head G = H_q / H_kv * L
SHAPES = [(2, 8, 2, 1), (1, 4, 1, 2), (1, 16, 2, 1)]


def _vid(v):
    return "D{}_g{}_v{}_{}{}{}".format(v[0], v[1], v[3], v[4], "_2s" if v[5] else "",
                                      "_rr" if v[6] else "")


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def _setup(var, dev, B, Hkv, T, seed):
    D, gs, kb, vb, dtype, two, rr = var
    tdt = W._TORCH_DTYPES[dtype]
    blocks = O.rotation_blocks(W.rotation_draws(seed, D), mode="two_sided" if two else "printed")
    if rr:
        blocks = O.round_to_dtype(blocks, dtype)
    rot = rbq.build_block_so4(D, seed, dev, two_sided=two, round_to=tdt if rr else None)
    c = rbq.RotatedQuantKVCache(B, Hkv, dtype=tdt, device=dev, rot=rot, head_dim=D,
                                group_size=gs, k_bits=kb, v_bits=vb, round_rotated=rr)
    oc = O.QuantKVCache(k_bits=kb, v_bits=vb, dtype=dtype, group=gs, round_rotated=rr)
    k = W.random_rows([seed, 1], (B, Hkv, T, D), dtype, "student_t3")
    v = W.random_rows([seed, 2], (B, Hkv, T, D), dtype)
    c.append(k.to(dev), v.to(dev))
    oc.append(k.float().numpy(), v.float().numpy(), blocks)
    return c, oc, blocks


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("var", VARS, ids=_vid)
def test_register_staged_tiles(var, splits, dev):
    D, dtype = var[0], var[4]
    T = 1000  # 31 whole tiles and 8 keys
    for si, (B, Hq, Hkv, L) in enumerate(SHAPES):
        print(f"[register tiles] {_vid(var)} splits={splits} B={B} Hq={Hq} Hkv={Hkv} L={L}",
              flush=True)
        c, oc, blocks = _setup(var, dev, B, Hkv, T, 40 + si)
        q = W.random_rows([41, si], (B, Hq, L, D), dtype)
        out = c.attend(q.to(dev), scale=D ** -0.5, causal=True, splits=splits)
        torch.cuda.synchronize()
        ref = O.attention(q.float().numpy(), oc, D ** -0.5, True, blocks)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= ATOL, (B, Hq, Hkv, L, err)


@pytest.mark.parametrize("splits", [0, 1])
def test_register_staged_tiles_masks(splits, dev):
    var = (128, 64, 4, 4, "bf16", True, False)
    B, Hq, Hkv, L, T = 2, 8, 2, 2, 777
    c, oc, blocks = _setup(var, dev, B, Hkv, T, 45)
    q = W.random_rows([46, 0], (B, Hq, L, 128), "bf16")
    rng = np.random.default_rng([46, 1])
    # additive mask (natural-log units), float32
    add = rng.normal(0.0, 2.0, size=(B, Hq, L, T)).astype(np.float32)
    out = c.attend(q.to(dev), scale=128 ** -0.5, causal=True, splits=splits,
                   mask=torch.from_numpy(add).to(dev))
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 128 ** -0.5, True, blocks, mask=add)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= ATOL, ("additive", err)
    # boolean mask; some rows keep no key (the mean of their keys' values)
    keep = rng.random(size=(B, Hq, L, T)) < 0.3
    keep[0, 1, 0, :] = False
    keep[1, 6, 1, :] = False
    out = c.attend(q.to(dev), scale=128 ** -0.5, causal=True, splits=splits,
                   mask=torch.from_numpy(keep).to(dev))
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 128 ** -0.5, True, blocks, mask=keep)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= ATOL, ("boolean", err)


@pytest.mark.parametrize("T", [1, 31, 32, 33, 65])
@pytest.mark.parametrize("splits", [0, 1, 7])
def test_register_staged_tiles_short_caches(T, splits, dev):
    # fewer keys than one tile, exactly one, one and a bit, two and a bit;
    # explicit splits beyond the tile count
    var = (128, 64, 4, 3, "bf16", True, False)
    B, Hq, Hkv, L = 1, 16, 2, 1
    print(f"[register tiles] short cache T={T} splits={splits}", flush=True)
    c, oc, blocks = _setup(var, dev, B, Hkv, T, 47)
    q = W.random_rows([48, T], (B, Hq, L, 128), "bf16")
    out = c.attend(q.to(dev), scale=128 ** -0.5, causal=True, splits=splits)
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 128 ** -0.5, True, blocks)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= ATOL, err


def test_register_staged_tiles_decode_steps(dev):
    # the one-call step on this configuration (the append kernel, then the
    # attention), several steps in a row over a growing cache
    var = (64, 32, 4, 4, "f16", False, False)
    B, Hq, Hkv, T0 = 2, 8, 2, 250
    c, oc, blocks = _setup(var, dev, B, Hkv, T0, 49)
    for step in range(4):
        kn = W.random_rows([50, step], (B, Hkv, 1, 64), "f16", "student_t3")
        vn = W.random_rows([51, step], (B, Hkv, 1, 64), "f16")
        q = W.random_rows([52, step], (B, Hq, 1, 64), "f16")
        out = c.append_attend(kn.to(dev), vn.to(dev), q.to(dev), scale=0.125, causal=True)
        torch.cuda.synchronize()
        oc.append(kn.float().numpy(), vn.float().numpy(), blocks)
        ref = O.attention(q.float().numpy(), oc, 0.125, True, blocks)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= ATOL, (step, err)

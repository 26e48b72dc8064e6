"""GPU parity of the tile kernel's staged single-wave shape with paired rows.

Calls with at most 8 query rows per kv head whose widths or head dim the
register-staged shape does not take (K codes other than 4 bits, V codes
above 4 bits, head_dim 256) decode each tile into LDS and pair the hi and
lo parts of the query rows in one matrix operand.  Covered
here: head_dim 64, 128 and 256, 1, 2, 4 and 8 groups per row, K and V widths
from 2 to 8 bits, both dtypes, both rotations and the page's rotation
precision; 1, 4 and 8 rows per kv head (GQA rows and causal verify rows), a
ragged last tile, one split, automatic and explicit splits; an additive mask
and a boolean mask with rows that keep no key.
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
    (128, 64, 8, 8, "bf16", True, False),
    (256, 32, 6, 5, "bf16", False, False),
    (64, 64, 2, 8, "f16", True, True),
    (128, 128, 3, 2, "f16", False, False),
    (128, 32, 5, 6, "bf16", False, True),
    (64, 32, 4, 5, "f16", False, False),
    (256, 64, 4, 4, "bf16", True, False),
    (256, 128, 4, 2, "f16", False, True),
]
# (B, H_q, H_kv, L): rows per kv head G = H_q / H_kv * L
SHAPES = [(2, 8, 2, 1), (1, 4, 1, 2), (1, 16, 2, 1), (1, 2, 2, 1)]


def _vid(v):
    return "D{}_g{}_k{}v{}_{}{}{}".format(v[0], v[1], v[2], v[3], v[4], "_2s" if v[5] else "",
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
def test_paired_rows_staged(var, splits, dev):
    D, dtype = var[0], var[4]
    T = 1000  # 31 whole tiles and 8 keys
    for si, (B, Hq, Hkv, L) in enumerate(SHAPES):
        print(f"[paired rows] {_vid(var)} splits={splits} B={B} Hq={Hq} Hkv={Hkv} L={L}",
              flush=True)
        c, oc, blocks = _setup(var, dev, B, Hkv, T, 60 + si)
        q = W.random_rows([61, si], (B, Hq, L, D), dtype)
        out = c.attend(q.to(dev), scale=D ** -0.5, causal=True, splits=splits)
        torch.cuda.synchronize()
        ref = O.attention(q.float().numpy(), oc, D ** -0.5, True, blocks)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= ATOL, (B, Hq, Hkv, L, err)


@pytest.mark.parametrize("splits", [0, 1])
@pytest.mark.parametrize("var", [(256, 32, 6, 5, "bf16", True, False),
                                 (256, 64, 4, 4, "bf16", True, False)], ids=_vid)
def test_paired_rows_staged_masks(var, splits, dev):
    B, Hq, Hkv, L, T = 2, 8, 2, 2, 555
    print(f"[paired rows] masks {_vid(var)} splits={splits}", flush=True)
    c, oc, blocks = _setup(var, dev, B, Hkv, T, 65)
    q = W.random_rows([66, 0], (B, Hq, L, 256), "bf16")
    rng = np.random.default_rng([66, 1])
    add = rng.normal(0.0, 2.0, size=(B, Hq, L, T)).astype(np.float32)
    out = c.attend(q.to(dev), scale=1 / 16, causal=True, splits=splits,
                   mask=torch.from_numpy(add).to(dev))
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 1 / 16, True, blocks, mask=add)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= ATOL, ("additive", err)
    keep = rng.random(size=(B, Hq, L, T)) < 0.3
    keep[0, 3, 1, :] = False
    keep[1, 4, 0, :] = False
    out = c.attend(q.to(dev), scale=1 / 16, causal=True, splits=splits,
                   mask=torch.from_numpy(keep).to(dev))
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 1 / 16, True, blocks, mask=keep)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= ATOL, ("boolean", err)


@pytest.mark.parametrize("T", [1, 31, 33])
def test_paired_rows_staged_short_caches(T, dev):
    var = (128, 64, 8, 8, "bf16", True, False)
    B, Hq, Hkv, L = 1, 16, 2, 1
    print(f"[paired rows] short cache T={T}", flush=True)
    c, oc, blocks = _setup(var, dev, B, Hkv, T, 67)
    q = W.random_rows([68, T], (B, Hq, L, 128), "bf16")
    for splits in (0, 7):
        out = c.attend(q.to(dev), scale=128 ** -0.5, causal=True, splits=splits)
        torch.cuda.synchronize()
        ref = O.attention(q.float().numpy(), oc, 128 ** -0.5, True, blocks)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= ATOL, (splits, err)

"""GPU parity at the benchmark's secondary shapes, in the launch configuration
it times (automatic key splits), against the oracle on sampled outputs:

- the prefill chunk: 2048 new tokens appended to a cache of 8192 (T = 10240),
  B=1, 16 q heads / 2 kv heads, then the attention of the chunk's 2048 query
  rows per head with the causal mask at the offset; head_dim 256 K4/V3 (the
  prefill kernel's 128-row blocks) and head_dim 128 K4/V4 with the two-sided
  rotation (the same kernel's head_dim-128 build); query rows sampled over heads
  and positions (first rows, block edges, last rows);
- the head_dim-128 decode: B=8, 16/2 heads, group 64, K4/V4, two-sided
  rotation, T=32768 (the tile kernel); whole (b, kv head) slabs sampled.

The inputs are drawn with the benchmark's seeds.  Cache rows of the sampled
slabs are compared bit for bit with the oracle's.
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


def _slab_rows_equal(c, oc, b, h, ob=0, oh=0):
    rows = c.rows()
    for name, oname in NAMES:
        got = rows[name][b, h].cpu()
        got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
        ref = oc.arrays[oname][ob, oh, :oc.offset]
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"b={b} h={h} {name}: {len(bad)} mismatches, first {bad[:3].tolist()}"


@pytest.mark.parametrize("D", [256, 128])
def test_prefill_chunk_sampled_rows(D, dev):
    print(f"[prefill chunk] head_dim {D}", flush=True)
    Hkv, Hq, T0, L = 2, 16, 8192, 2048
    two = D != 256
    cfg = {} if D == 256 else dict(head_dim=D, group_size=64, k_bits=4, v_bits=4)
    blocks = O.rotation_blocks(W.rotation_draws(0, D), mode="two_sided" if two else "printed")
    rot = rbq.build_block_so4(D, 0, dev, two_sided=two)
    np.testing.assert_array_equal(rot.cpu().numpy(), blocks)
    k = W.random_rows([50, 1], (1, Hkv, T0, D), "bf16")
    v = W.random_rows([50, 2], (1, Hkv, T0, D), "bf16")
    kn = W.random_rows([50, 3], (1, Hkv, L, D), "bf16")
    vn = W.random_rows([50, 4], (1, Hkv, L, D), "bf16")
    q = W.random_rows([50, 5], (1, Hq, L, D), "bf16")
    c = rbq.RotatedQuantKVCache(1, Hkv, device=dev, rot=rot, **cfg)
    c.append(k.to(dev), v.to(dev))
    c.append(kn.to(dev), vn.to(dev))
    out = c.attend(q.to(dev), scale=D ** -0.5, causal=True)
    torch.cuda.synchronize()
    oc = O.QuantKVCache(k_bits=4, v_bits=3 if D == 256 else 4, dtype="bf16", group=64)
    oc.append(k.float().numpy(), v.float().numpy(), blocks)
    oc.append(kn.float().numpy(), vn.float().numpy(), blocks)
    for h in range(Hkv):
        _slab_rows_equal(c, oc, 0, h, 0, h)
    rng = np.random.default_rng([50, 9])
    pos = sorted(set([0, 1, 7, 8, 63, 64, 1000, L - 2, L - 1]) |
                 set(rng.integers(0, L, 6).tolist()))
    rows = [(0, h, i) for h in (0, 5, 8, 15) for i in pos]
    want = O.attention(q.float().numpy(), oc, D ** -0.5, True, blocks, rows=rows)
    got = out.cpu().numpy()
    for (b, h, i) in rows:
        err = float(np.abs(got[b, h, i] - want[b, h, i]).max())
        assert err <= ATOL, f"row (h={h}, i={i}): max abs error {err}"


def test_head_dim_128_decode_sampled_slabs(dev):
    print("[head_dim 128 decode] T=32768", flush=True)
    B, Hkv, Hq, T, D, gs, kb, vb = 8, 2, 16, 32768, 128, 64, 4, 4
    n_rep = Hq // Hkv
    blocks = O.rotation_blocks(W.rotation_draws(0, D), mode="two_sided")
    rot = rbq.build_block_so4(D, 0, dev, two_sided=True)
    k = W.random_rows([60, 1], (B, Hkv, T, D), "bf16")
    v = W.random_rows([60, 2], (B, Hkv, T, D), "bf16")
    c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot, head_dim=D, group_size=gs,
                                k_bits=kb, v_bits=vb)
    c.append(k.to(dev), v.to(dev))
    q = W.random_rows([60, 3], (B, Hq, 1, D), "bf16")
    out = c.attend(q.to(dev), scale=D ** -0.5, causal=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for (b, h) in ((0, 0), (3, 1), (7, 1)):
        print(f"  slab b={b} h={h}", flush=True)
        oc = O.QuantKVCache(k_bits=kb, v_bits=vb, dtype="bf16", group=gs)
        oc.append(k[b:b + 1, h:h + 1].float().numpy(), v[b:b + 1, h:h + 1].float().numpy(),
                  blocks)
        _slab_rows_equal(c, oc, b, h)
        qs = q[b:b + 1, h * n_rep:(h + 1) * n_rep].float().numpy()
        want = O.attention(qs, oc, D ** -0.5, True, blocks)
        err = float(np.abs(got[b, h * n_rep:(h + 1) * n_rep] - want[0]).max())
        assert err <= ATOL, f"slab b={b} h={h}: max abs error {err}"

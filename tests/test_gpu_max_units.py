"""GPU: more (b, kv head) slabs than one grid dimension takes.

The dedicated kernel and the prefill kernel put the (b, kv head) slabs on
grid z, at most 65535 workgroups per launch, and launch the rest with an
offset.  Here B = 65537 slabs of one kv head each: a decode (one key per
slab after a one-token append, 8-row blocks) and a prefill block of 96 rows
per slab (the prefill kernel), checked against the oracle on slabs on both
sides of the 65535 boundary and at the ends.  The bulk inputs are drawn on
the device from a seeded generator; the oracle sees the sampled slabs only
(slabs are independent).
"""
import numpy as np
import pytest
import torch

from oracle import rbq_oracle as O
import workloads as W

pytestmark = pytest.mark.gpu

ATOL = 2e-3
rbq = pytest.importorskip("rotated_bit_quantized_amd")

B = 65537
SAMPLE = (0, 1, 65533, 65534, 65535, 65536)


@pytest.mark.parametrize("T,L", [(1, 1), (96, 96)], ids=["decode_8row_blocks", "prefill_96_rows"])
def test_slabs_past_one_grid_dimension(T, L):
    dev = torch.device("cuda:0")
    print(f"[max units] B={B} T={T} L={L}", flush=True)
    blocks = O.rotation_blocks(W.rotation_draws(4, 256))
    rot = rbq.build_block_so4(256, 4, dev)
    g = torch.Generator(device=dev).manual_seed(1234 + T)
    k = torch.randn(B, 1, T, 256, generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn(B, 1, T, 256, generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn(B, 1, L, 256, generator=g, device=dev).to(torch.bfloat16)
    c = rbq.RotatedQuantKVCache(B, 1, device=dev, rot=rot)
    c.append(k, v)
    out = c.attend(q, scale=1 / 16, causal=True)
    torch.cuda.synchronize()
    for b in SAMPLE:
        oc = O.QuantKVCache(k_bits=4, v_bits=3, dtype="bf16", group=64)
        oc.append(k[b:b + 1].float().cpu().numpy(), v[b:b + 1].float().cpu().numpy(), blocks)
        ref = O.attention(q[b:b + 1].float().cpu().numpy(), oc, 1 / 16, True, blocks)
        err = float(np.abs(out[b:b + 1].cpu().numpy() - ref).max())
        assert err <= ATOL, (b, err)
    del c, k, v, q, out
    torch.cuda.empty_cache()

"""GPU: the attention entry point that allocates nothing
(rbq_quant_attn_decode_noalloc, split records in the library's fixed device
array) against rbq_quant_attn_decode with a workspace, through the C ABI:
two calls in a row, the second on a smaller input, each output bit for bit
that of the workspace call (same kernels, same split plan) and within the
tolerance of the oracle, for the 8-row blocks, the tile kernel and the
prefill kernel's split records; and a call that needs more than the fixed
array is refused before anything is launched."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O

pytestmark = pytest.mark.gpu

ATOL = 2e-3
rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402


def _cache(dev, seed, B, Hkv, T, blocks, rot, **cfg):
    D = cfg.get("head_dim", 256)
    c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot, **cfg)
    oc = O.QuantKVCache(k_bits=cfg.get("k_bits", 4), v_bits=cfg.get("v_bits", 3), dtype="bf16",
                        group=cfg.get("group_size", 64))
    k = W.random_rows([seed, 1], (B, Hkv, T, D), "bf16")
    v = W.random_rows([seed, 2], (B, Hkv, T, D), "bf16")
    c.append(k.to(dev), v.to(dev))
    oc.append(k.float().numpy(), v.float().numpy(), blocks)
    return c, oc


@pytest.mark.parametrize("D", [256, 128])
def test_noalloc_matches_the_workspace_call_twice(D):
    dev = torch.device("cuda:0")
    print(f"[no-alloc attention] head_dim {D}", flush=True)
    cfg = {} if D == 256 else dict(head_dim=D, group_size=64, k_bits=4, v_bits=4)
    blocks = O.rotation_blocks(W.rotation_draws(0, D))
    rot = rbq.build_block_so4(D, 0, dev)
    # first call: many splits (split records in the array); second: a smaller
    # cache, fewer query rows, its records overwrite the first call's
    shapes = [(2, 16, 2, 5000, 2, 0), (1, 8, 2, 700, 1, 3)]
    for n, (B, Hq, Hkv, T, L, splits) in enumerate(shapes):
        c, oc = _cache(dev, 90 + n, B, Hkv, T, blocks, rot, **cfg)
        q = W.random_rows([90 + n, 3], (B, Hq, L, D), "bf16").to(dev)
        need = capi.rbq_quant_attn_workspace_bytes(c.desc, Hq, L, splits)
        assert 0 < need <= capi.RBQ_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        want = torch.empty(q.shape, dtype=torch.float32, device=dev)
        got = torch.full(q.shape, float("nan"), dtype=torch.float32, device=dev)
        capi.rbq_quant_attn_decode(c.desc, q, D ** -0.5, True, rot, want, splits, ws)
        capi.rbq_quant_attn_decode_noalloc(c.desc, q, D ** -0.5, True, rot, got, splits)
        torch.cuda.synchronize()
        assert torch.equal(got, want), float((got - want).abs().max())
        ref = O.attention(q.cpu().float().numpy(), oc, D ** -0.5, True, blocks)
        assert float(np.abs(got.cpu().numpy() - ref).max()) <= ATOL


@pytest.mark.parametrize("D", [256, 64])
def test_noalloc_prefill_kernel_records_then_a_smaller_call(D):
    # 128 query rows per kv head (the prefill kernel) over few (b, kv head)
    # units: key splits whose records go to the array; then a call of 48
    # rows (8-row blocks at head_dim 256, the tile kernel at 64) whose records
    # overwrite the first call's
    dev = torch.device("cuda:0")
    print(f"[no-alloc attention] prefill kernel, head_dim {D}", flush=True)
    cfg = {} if D == 256 else dict(head_dim=D, group_size=64, k_bits=4, v_bits=4)
    blocks = O.rotation_blocks(W.rotation_draws(1, D))
    rot = rbq.build_block_so4(D, 1, dev)
    shapes = [(1, 16, 2, 3000, 16), (1, 8, 2, 900, 12)]
    for n, (B, Hq, Hkv, T, L) in enumerate(shapes):
        c, oc = _cache(dev, 95 + n, B, Hkv, T, blocks, rot, **cfg)
        q = W.random_rows([95 + n, 3], (B, Hq, L, D), "bf16").to(dev)
        assert capi.rbq_quant_attn_splits(c.desc, Hq, L) > 1
        need = capi.rbq_quant_attn_workspace_bytes(c.desc, Hq, L, 0)
        assert 0 < need <= capi.RBQ_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        want = torch.empty(q.shape, dtype=torch.float32, device=dev)
        got = torch.full(q.shape, float("nan"), dtype=torch.float32, device=dev)
        capi.rbq_quant_attn_decode(c.desc, q, 1 / 16, True, rot, want, 0, ws)
        capi.rbq_quant_attn_decode_noalloc(c.desc, q, 1 / 16, True, rot, got, 0)
        torch.cuda.synchronize()
        assert torch.equal(got, want), float((got - want).abs().max())
        ref = O.attention(q.cpu().float().numpy(), oc, 1 / 16, True, blocks)
        assert float(np.abs(got.cpu().numpy() - ref).max()) <= ATOL


def test_noalloc_refuses_more_than_the_array():
    dev = torch.device("cuda:0")
    # a descriptor only (no device work happens): enough (b, kv head) units
    # and splits that the split records exceed the fixed array
    c = rbq.RotatedQuantKVCache(64, 8, device=dev)
    c.reserve(8192)
    c.desc.offset = 8192
    q = torch.zeros((64, 64, 1, 256), dtype=torch.bfloat16, device=dev)
    out = torch.zeros(q.shape, dtype=torch.float32, device=dev)
    need = capi.rbq_quant_attn_workspace_bytes(c.desc, 64, 1, 32)
    assert need > capi.RBQ_SCRATCH_BYTES
    with pytest.raises(capi.RbqError) as e:
        capi.rbq_quant_attn_decode_noalloc(c.desc, q, 1 / 16, True, None, out, 32)
    assert e.value.status == capi.RBQ_ESCRATCH
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0

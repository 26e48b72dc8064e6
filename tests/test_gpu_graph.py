"""GPU: the decode step (append one token, attend; as two calls and as the
one-call step) captured in a HIP graph, and attention calls of the prefill
kernel, the tile kernel and the entry point that allocates nothing captured
the same way.

The launches read their arguments as captured: a replay appends the token at
the captured row again and attends over the same rows, so every replay must
reproduce the eager step's output exactly (the kernels are deterministic: a
fixed split plan and a fixed merge order).  The replays are interleaved with
eager work on another cache and with synchronisations, and each replay is
checked, as graph replays of the same step are used by the benchmark.
"""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402


def _cache(dev, rot, B, Hkv, T, seed):
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(B, Hkv, T, 256, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, T, 256, generator=g).to(torch.bfloat16)
    c = rbq.RotatedQuantKVCache(B, Hkv, dtype=torch.bfloat16, device=dev, rot=rot)
    c.append(k.to(dev), v.to(dev))
    return c


@pytest.mark.parametrize("one_call", [False, True], ids=["two_calls", "one_call"])
@pytest.mark.parametrize("T", [300, 5000])
def test_step_graph_replays_equal_eager(T, one_call):
    dev = torch.device("cuda:0")
    rot = rbq.build_block_so4(256, W.ROTATION_SEED, dev)
    B, Hkv, Hq = 2, 2, 16
    print(f"graph step B={B} Hq={Hq} Hkv={Hkv} T={T} one_call={one_call}", flush=True)
    c = _cache(dev, rot, B, Hkv, T - 1, 1)
    other = _cache(dev, rot, B, Hkv, T, 2)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(B, Hq, 1, 256, generator=g).to(torch.bfloat16).to(dev)
    k1 = torch.randn(B, Hkv, 1, 256, generator=g).to(torch.bfloat16).to(dev)
    v1 = torch.randn(B, Hkv, 1, 256, generator=g).to(torch.bfloat16).to(dev)
    out = torch.empty(B, Hq, 1, 256, dtype=torch.float32, device=dev)
    out_other = torch.empty_like(out)
    ws = c.workspace(Hq, 1)
    ws_other = torch.zeros_like(ws) if ws is not None else None

    def step():
        if one_call:  # the attention kernel appends the token itself
            capi.rbq_kv_append_attn_decode(c.desc, k1, v1, q, 1 / 16, True, rot, out, 0, ws)
            return
        capi.rbq_kv_quant_append(c.desc, k1, v1, rot)
        capi.rbq_quant_attn_decode(c.desc, q, 1 / 16, True, rot, out, 0, ws)

    # eager reference
    step()
    torch.cuda.synchronize()
    want = out.clone()
    words = c.arrays["k_words"][:, :, T - 1].clone()
    capi.rbq_kv_trim(c.desc, 1)

    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    out.zero_()
    with torch.cuda.graph(graph, stream=cap):
        step()
    capi.rbq_kv_trim(c.desc, 1)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        c.arrays["k_words"][:, :, T - 1].zero_()
        graph.replay()
        # eager work on another cache between replays
        capi.rbq_quant_attn_decode(other.desc, q, 1 / 16, True, rot, out_other, 0, ws_other)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}: output differs from the eager step"
        assert torch.equal(c.arrays["k_words"][:, :, T - 1], words), f"replay {r}: appended row"


# (kind, head_dim, group, k_bits, v_bits, B, H_q, H_kv, T, L): attention calls
# of the other kernels captured the same way: the prefill kernel with key
# splits and the record merge (128 rows per kv head), the tile kernel (a
# head_dim-128 K4/V4 decode, register-staged tiles, and a long block of a
# 5/6-bit layout, four-wave tiles) and the entry point that allocates nothing
# (its records in the library's fixed array) on the 8-row blocks and on the
# prefill kernel
GRAPH_CALLS = [
    ("prefill", 256, 64, 4, 3, 1, 16, 2, 3000, 16),
    ("tile_decode", 128, 64, 4, 4, 2, 16, 2, 4000, 1),
    ("tile_block", 128, 32, 5, 6, 1, 8, 2, 900, 24),
    ("noalloc_decode", 256, 64, 4, 3, 2, 16, 2, 5000, 1),
    ("noalloc_prefill", 256, 64, 4, 3, 1, 16, 2, 3000, 16),
]


@pytest.mark.parametrize("case", GRAPH_CALLS, ids=[c[0] for c in GRAPH_CALLS])
def test_attention_graph_replays_equal_eager(case):
    kind, D, gs, kb, vb, B, Hq, Hkv, T, L = case
    dev = torch.device("cuda:0")
    print(f"graph attention {kind}: D={D} g{gs} k{kb}v{vb} B={B} Hq={Hq} Hkv={Hkv} T={T} L={L}",
          flush=True)
    rot = rbq.build_block_so4(D, W.ROTATION_SEED, dev)
    g = torch.Generator().manual_seed(11)
    k = torch.randn(B, Hkv, T, D, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, T, D, generator=g).to(torch.bfloat16)
    c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot, head_dim=D, group_size=gs,
                                k_bits=kb, v_bits=vb)
    c.append(k.to(dev), v.to(dev))
    other = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot, head_dim=D, group_size=gs,
                                    k_bits=kb, v_bits=vb)
    other.append(v.to(dev), k.to(dev))
    q = torch.randn(B, Hq, L, D, generator=g).to(torch.bfloat16).to(dev)
    out = torch.empty(B, Hq, L, D, dtype=torch.float32, device=dev)
    out_other = torch.empty_like(out)
    noalloc = kind.startswith("noalloc")
    assert capi.rbq_quant_attn_splits(c.desc, Hq, L) > 1
    ws = None if noalloc else c.workspace(Hq, L)
    ws_other = None if noalloc else torch.zeros_like(ws)
    scale = D ** -0.5

    def call(cache, o, w):
        if noalloc:
            capi.rbq_quant_attn_decode_noalloc(cache.desc, q, scale, True, rot, o, 0)
        else:
            capi.rbq_quant_attn_decode(cache.desc, q, scale, True, rot, o, 0, w)

    call(c, out, ws)
    torch.cuda.synchronize()
    want = out.clone()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    out.zero_()
    with torch.cuda.graph(graph, stream=cap):
        call(c, out, ws)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        graph.replay()
        # eager work between replays (with the fixed array: the same array)
        call(other, out_other, ws_other)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}: output differs from the eager call"

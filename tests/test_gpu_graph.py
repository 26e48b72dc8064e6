"""GPU: the decode step (append one token, attend; as two calls and as the
one-call step) captured in a HIP graph.

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

"""GPU: one workspace shared by back-to-back attention calls of different
shapes.  Calls with different queries, caches and split counts are
interleaved on one workspace that holds arbitrary bytes before the first
call, so that a split record left by an earlier call would show: every
output is checked against the oracle, and repeats of one call against each
other bit for bit; split counts on either side of 32 agree."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O

pytestmark = pytest.mark.gpu

ATOL = 2e-3
rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402


def test_interleaved_calls_share_one_workspace():
    dev = torch.device("cuda:0")
    print("[fused merge] interleaved calls", flush=True)
    blocks = O.rotation_blocks(W.rotation_draws(0, 256))
    rot = rbq.build_block_so4(256, 0, dev)
    B, Hkv, Hq = 2, 2, 16
    caches, ocs = [], []
    for seed, T in ((101, 3000), (102, 6000)):
        k = W.random_rows([seed, 1], (B, Hkv, T, 256), "bf16")
        v = W.random_rows([seed, 2], (B, Hkv, T, 256), "bf16", "student_t3")
        c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
        c.append(k.to(dev), v.to(dev))
        oc = O.QuantKVCache(dtype="bf16")
        oc.append(k.float().numpy(), v.float().numpy(), blocks)
        caches.append(c)
        ocs.append(oc)
    qs = [W.random_rows([103, i], (B, Hq, L, 256), "bf16") for i, L in enumerate((1, 1, 2))]
    # cases: (cache, query, splits)
    cases = [(ci, qi, sp) for ci in range(2) for qi in range(3) for sp in (0, 3, 16, 32)]
    nb = max(capi.rbq_quant_attn_workspace_bytes(caches[ci].desc, Hq, qs[qi].shape[2], sp)
             for ci, qi, sp in cases)
    assert nb > 0
    ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device=dev)  # arbitrary bytes first
    want = {}
    for ci in range(2):
        for qi in range(3):
            want[ci, qi] = O.attention(qs[qi].float().numpy(), ocs[ci], 1 / 16, True, blocks)
    qd = [q.to(dev) for q in qs]
    first = {}
    rng = np.random.default_rng(104)
    for r in range(6):
        order = rng.permutation(len(cases))
        outs = []
        for idx in order:
            ci, qi, sp = cases[idx]
            out = torch.empty(qs[qi].shape, dtype=torch.float32, device=dev)
            capi.rbq_quant_attn_decode(caches[ci].desc, qd[qi], 1 / 16, True, rot, out, sp, ws)
            outs.append((cases[idx], out))
        torch.cuda.synchronize()
        for (ci, qi, sp), out in outs:
            got = out.cpu()
            err = float(np.abs(got.numpy() - want[ci, qi]).max())
            assert err <= ATOL, (r, ci, qi, sp, err)
            key = (ci, qi, sp)
            if key in first:
                assert torch.equal(got, first[key]), (r, key)
            else:
                first[key] = got


def test_split_counts_around_the_fused_limit_agree():
    # 31, 32, 33 and 40 splits of the same call (one, two or three rounds of
    # 16 records in the merge kernel): within the tolerance of each other and
    # of the oracle
    dev = torch.device("cuda:0")
    blocks = O.rotation_blocks(W.rotation_draws(0, 256))
    rot = rbq.build_block_so4(256, 0, dev)
    B, Hkv, Hq, T = 1, 2, 16, 9000
    k = W.random_rows([105, 1], (B, Hkv, T, 256), "bf16")
    v = W.random_rows([105, 2], (B, Hkv, T, 256), "bf16")
    c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
    c.append(k.to(dev), v.to(dev))
    oc = O.QuantKVCache(dtype="bf16")
    oc.append(k.float().numpy(), v.float().numpy(), blocks)
    q = W.random_rows([105, 3], (B, Hq, 1, 256), "bf16")
    outs = [c.attend(q.to(dev), scale=1 / 16, causal=True, splits=sp) for sp in (31, 32, 33, 40)]
    torch.cuda.synchronize()
    want = O.attention(q.float().numpy(), oc, 1 / 16, True, blocks)
    for o in outs:
        assert float(np.abs(o.cpu().numpy() - want).max()) <= ATOL
        assert float((o - outs[0]).abs().max()) <= 1e-5

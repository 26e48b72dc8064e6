"""GPU: every build of the split-record merge against the oracle.

The merge of the dedicated kernel's records comes in six builds: 32 or 64
columns per workgroup (fewer or at least 64 (b, kv head, 8-row) units) and
one, two or four groups of 128 threads (up to 16, up to 32, more splits).
Each is reached here by the unit count and an explicit split count, on the
default layout, with the causal mask and with a boolean mask that leaves one
row without a kept key (the merge then takes the mean of that row's keys).
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O

pytestmark = pytest.mark.gpu

ATOL = 2e-3
rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402

# (B, H_q, H_kv, L, T, splits, groups): units = B * H_kv * ceil(H_q / H_kv *
# L / 8); with one 8-row block per kv head a split holds whole 256-key
# rounds, with several whole 32-key tiles
CASES = [
    (1, 16, 2, 1, 9000, 12, 1),   # 2 units: 32 columns, one group
    (1, 16, 2, 1, 9000, 24, 2),   # two groups
    (1, 16, 2, 1, 9000, 36, 4),   # four groups
    (4, 32, 4, 4, 3000, 16, 1),   # 64 units: 64 columns, one group
    (4, 32, 4, 4, 3000, 32, 2),   # two groups
    (4, 32, 4, 4, 3000, 48, 4),   # four groups
]
REC_BYTES = (2 * 8 + 8 * 256) * 4  # one split record of 8 rows


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_H{}-{}_L{}_T{}_s{}".format(*c[:6]))
@pytest.mark.parametrize("masked", [False, True], ids=["causal", "bool_mask"])
def test_merge_builds(case, masked):
    B, Hq, Hkv, L, T, splits, groups = case
    dev = torch.device("cuda:0")
    print(f"[merge builds] B={B} Hq={Hq} Hkv={Hkv} L={L} splits={splits} masked={masked}", flush=True)
    blocks = O.rotation_blocks(W.rotation_draws(3, 256))
    rot = rbq.build_block_so4(256, 3, dev)
    c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
    oc = O.QuantKVCache(k_bits=4, v_bits=3, dtype="bf16", group=64)
    k = W.random_rows([97, 1], (B, Hkv, T, 256), "bf16", "student_t3")
    v = W.random_rows([97, 2], (B, Hkv, T, 256), "bf16")
    c.append(k.to(dev), v.to(dev))
    oc.append(k.float().numpy(), v.float().numpy(), blocks)
    units = B * Hkv * ((Hq // Hkv * L + 7) // 8)
    S = capi.rbq_quant_attn_workspace_bytes(c.desc, Hq, L, splits) // (units * REC_BYTES)
    assert (S <= 16, 16 < S <= 32, S > 32)[{1: 0, 2: 1, 4: 2}[groups]], S
    q = W.random_rows([97, 3], (B, Hq, L, 256), "bf16")
    m_np = m_dev = None
    if masked:
        rng = np.random.default_rng([97, 4])
        m_np = rng.random(size=(B, Hq, L, T)) < 0.4
        m_np[B - 1, Hq - 1, L - 1, :] = False
        m_dev = torch.from_numpy(m_np).to(dev)
    out = c.attend(q.to(dev), scale=1 / 16, causal=True, splits=splits, mask=m_dev)
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, 1 / 16, True, blocks, mask=m_np)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= ATOL, err

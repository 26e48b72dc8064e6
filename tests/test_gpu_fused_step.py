"""GPU parity of the one-call decoding step through the C ABI
(rbq_kv_append_attn_decode: the append of n rows followed by the attention
over the cache that results).  Where the attention kernel writes the rows
itself, the cache rows and the output must equal those of the two calls
(rbq_kv_quant_append, then rbq_quant_attn_decode) bit for bit, and the oracle
within the attention tolerance; the shapes cover appended rows in the last
tile of a long split, rows that straddle two key splits, rows inside the
first tile of a workgroup (whose transfer then waits for them), one split
with the output stored directly, several blocks of query rows per kv head
(every block's workgroups write the rows of their split), no rotation, the
page's rotation precision, fp16, and the shape that runs as two launches.
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

NAMES = (("k_words", "kw"), ("k_scales", "ks"), ("k_biases", "kb"),
         ("v_words", "vw"), ("v_scales", "vs"), ("v_biases", "vb"))

# dtype, round_rotated, rotated, B, H_q, H_kv, cached rows, n appended, L, splits
CASES = [
    ("bf16", False, True, 2, 16, 2, 1000, 1, 1, 0),    # decode, automatic splits
    ("bf16", False, True, 2, 16, 2, 4095, 1, 1, 1),    # one split: output stored directly
    ("f16", True, True, 1, 4, 2, 59, 8, 4, 2),         # rows 59-66 straddle splits [0,64) [64,67)
    ("bf16", False, False, 2, 2, 2, 2, 8, 8, 0),       # T = 10: appended rows in the first tile
    ("bf16", True, True, 1, 16, 2, 256, 1, 1, 0),      # the append grows the buffers first
    ("f16", False, True, 1, 8, 1, 700, 1, 1, 3),       # explicit splits, one kv head
    ("bf16", False, True, 1, 16, 2, 300, 2, 2, 0),     # 16 rows per kv head (two row blocks)
    ("bf16", False, True, 4, 16, 2, 10240, 4, 4, 0),   # the verify block: 32 rows, 4 row blocks
    ("f16", True, True, 2, 16, 2, 507, 6, 4, 5),       # 4 row blocks, rows 507-512 straddle
                                                       # the splits [384, 512) and [512, 513)
    ("bf16", False, True, 1, 16, 2, 300, 9, 1, 0),     # 9 rows appended: two launches
]


def _cid(c):
    return "{}{}{}_B{}_H{}-{}_T{}_n{}_L{}_S{}".format(c[0], "_rr" if c[1] else "",
                                                      "" if c[2] else "_norot", *c[3:])


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


def _caches(case, dev, seed):
    dtype, rr, rotated, B, Hq, Hkv, T0, n, L, _ = case
    tdt = W._TORCH_DTYPES[dtype]
    D = 256
    if rotated:
        blocks = O.rotation_blocks(W.rotation_draws(seed, D))
        if rr:
            blocks = O.round_to_dtype(blocks, dtype)
        rot = rbq.build_block_so4(D, seed, dev, round_to=tdt if rr else None)
        np.testing.assert_array_equal(rot.cpu().numpy(), blocks)
    else:
        blocks, rot = None, None
    k = W.random_rows([seed, 1], (B, Hkv, T0 + n, D), dtype, "student_t3")
    v = W.random_rows([seed, 2], (B, Hkv, T0 + n, D), dtype)
    q = W.random_rows([seed, 3], (B, Hq, L, D), dtype)
    caches = []
    for _ in range(2):
        c = rbq.RotatedQuantKVCache(B, Hkv, dtype=tdt, device=dev, rot=rot, round_rotated=rr)
        c.append(k[:, :, :T0].contiguous().to(dev), v[:, :, :T0].contiguous().to(dev))
        caches.append(c)
    oc = O.QuantKVCache(k_bits=4, v_bits=3, dtype=dtype, group=64, round_rotated=rr)
    oc.append(k[:, :, :T0].float().numpy(), v[:, :, :T0].float().numpy(), blocks)
    new = (k[:, :, T0:].contiguous(), v[:, :, T0:].contiguous())
    return caches, oc, blocks, new, q


def _rows(c):
    torch.cuda.synchronize()
    return {name: c.rows()[name].cpu() for name, _ in NAMES}


@pytest.mark.parametrize("case", CASES, ids=_cid)
def test_fused_step_matches_two_calls_and_oracle(case, dev):
    print(f"[fused step] {_cid(case)}", flush=True)
    splits = case[9]
    (c1, c2), oc, blocks, (kn, vn), q = _caches(case, dev, 21)
    qd = q.to(dev)
    out1 = c1.append_attend(kn.to(dev), vn.to(dev), qd, scale=1 / 16, causal=True, splits=splits)
    c2.append(kn.to(dev), vn.to(dev))
    out2 = c2.attend(qd, scale=1 / 16, causal=True, splits=splits)
    torch.cuda.synchronize()
    assert (c1.offset, c1.capacity) == (c2.offset, c2.capacity)
    r1, r2 = _rows(c1), _rows(c2)
    for name, _ in NAMES:
        assert torch.equal(r1[name], r2[name]), name
    assert torch.equal(out1, out2), float((out1 - out2).abs().max())
    # the oracle: the same rows bit for bit, the output within the tolerance
    oc.append(kn.float().numpy(), vn.float().numpy(), blocks)
    assert c1.offset == oc.offset
    for name, oname in NAMES:
        got = r1[name]
        got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
        bad = np.argwhere(got != oc.arrays[oname][:, :, :oc.offset])
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
    ref = O.attention(q.float().numpy(), oc, 1 / 16, True, blocks)
    err = float(np.abs(out1.cpu().numpy() - ref).max())
    assert err <= ATOL, err


def test_fused_steps_overwrite_the_same_row(dev):
    # the decode loop of the benchmark: append one token and attend, trim it,
    # again with another token at the same row; every step must read the row
    # it has just written, not an earlier one
    case = ("bf16", False, True, 2, 16, 2, 2047, 1, 1, 0)
    print("[fused step] same row, new tokens", flush=True)
    (c, _), oc, blocks, _, q = _caches(case, dev, 22)
    qd = q.to(dev)
    B, Hkv = 2, 2
    for step in range(4):
        kn = W.random_rows([22, 10 + step], (B, Hkv, 1, 256), "bf16", "student_t3", scale=3.0)
        vn = W.random_rows([22, 20 + step], (B, Hkv, 1, 256), "bf16", scale=3.0)
        out = c.append_attend(kn.to(dev), vn.to(dev), qd, scale=1 / 16, causal=True)
        torch.cuda.synchronize()
        oc.append(kn.float().numpy(), vn.float().numpy(), blocks)
        ref = O.attention(q.float().numpy(), oc, 1 / 16, True, blocks)
        err = float(np.abs(out.cpu().numpy() - ref).max())
        assert err <= ATOL, (step, err)
        row = c.rows()
        for name, oname in NAMES:
            got = row[name][:, :, -1:].cpu()
            got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
            assert np.array_equal(got, oc.arrays[oname][:, :, oc.offset - 1:oc.offset]), \
                (step, name)
        assert c.trim(1) == 1
        oc.trim(1)


def test_fused_step_n0_is_the_attention(dev):
    case = ("bf16", False, True, 1, 16, 2, 500, 1, 1, 0)
    (c1, c2), _, _, _, q = _caches(case, dev, 23)
    qd = q.to(dev)
    empty = torch.empty((1, 2, 0, 256), dtype=torch.bfloat16, device=dev)
    out1 = c1.append_attend(empty, empty, qd, scale=1 / 16)
    out2 = c2.attend(qd, scale=1 / 16)
    torch.cuda.synchronize()
    assert c1.offset == 500
    assert torch.equal(out1, out2)


def test_prepared_step_equals_the_binding_call(dev):
    # the step with its arguments marshalled once (the benchmark's loop) makes
    # the same library call: rows and output bit for bit
    case = ("bf16", False, True, 2, 16, 2, 777, 1, 1, 0)
    print("[fused step] prepared call", flush=True)
    (c1, c2), _, _, (kn, vn), q = _caches(case, dev, 24)
    kd, vd, qd = kn.to(dev), vn.to(dev), q.to(dev)
    after = capi.rbq_kv_cache.from_buffer_copy(c1.desc)
    after.offset += 1
    nb = capi.rbq_quant_attn_workspace_bytes(after, 16, 1, 0)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    out1 = torch.empty(qd.shape, dtype=torch.float32, device=dev)
    out2 = torch.empty_like(out1)
    c1.reserve(1)
    c2.reserve(1)
    call = capi.prepare_append_attn_decode(c1.desc, kd, vd, qd, 1 / 16, True, c1.rot, out1, 0, ws)
    call(c1.desc)
    capi.rbq_kv_append_attn_decode(c2.desc, kd, vd, qd, 1 / 16, True, c2.rot, out2, 0, ws)
    torch.cuda.synchronize()
    assert c1.offset == c2.offset
    assert torch.equal(out1, out2)
    r1, r2 = _rows(c1), _rows(c2)
    for name, _ in NAMES:
        assert torch.equal(r1[name], r2[name]), name

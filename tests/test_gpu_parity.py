"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Quantize/pack: packed words, scales and biases bit for bit.  Attention:
within 2e-3 max abs (fp32 accumulation on the GPU, fp64 in the oracle).
Workloads: the five synthetic workloads of ``workloads.WORKLOADS`` at their
full sizes (every (batch, kv head) slab whole), and small ragged /
degenerate cases.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import rbq_oracle as O
import _ref as R

pytestmark = pytest.mark.gpu

ATOL = 2e-3

rbq = pytest.importorskip("rotated_bit_quantized_amd")
from rotated_bit_quantized_amd import capi  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def blocks():
    return O.rotation_blocks(W.rotation_draws(W.ROTATION_SEED, 256))


@pytest.fixture(scope="module")
def rot(dev):
    return rbq.build_block_so4(256, W.ROTATION_SEED, dev)


def test_device_rotation_blocks_equal_oracle(rot, blocks):
    np.testing.assert_array_equal(rot.cpu().numpy(), blocks)


def _fill(w, dev, rot, k, v):
    c = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
    c.append(k.to(dev), v.to(dev))
    return c


def _check_slab(c, k, v, b, h, blocks, dtype, rows=None):
    kk = k[b, h].float().numpy()
    vv = v[b, h].float().numpy()
    if rows is not None:
        kk, vv = kk[rows], vv[rows]
    ref = R.oracle_rows(kk, vv, blocks, dtype)
    got = R.device_rows(c, b, h, rows)
    R.assert_slab_equal(got, ref, f"slab b={b} h={h}")
    return ref


def _check_attention(c, q, out, b, kvh, ref, blocks, causal, what=""):
    khat, vhat = R.dequant_slab(ref)
    n_rep = q.shape[1] // c.desc.H_kv
    want = R.oracle_attention_slab(q.float().numpy(), b, kvh, n_rep, khat, vhat, c.offset,
                                   causal, blocks, 1 / 16)
    got = out[b, kvh * n_rep:(kvh + 1) * n_rep].cpu().numpy()
    err = float(np.abs(got - want).max())
    assert err <= ATOL, f"{what} b={b} kvh={kvh}: max abs error {err}"
    return err


# ------------------------------------------------------------- workloads --

@pytest.mark.parametrize("cid", [1, 2])
def test_small_workloads_full(cid, dev, rot, blocks):
    w = W.WORKLOADS[cid]
    print(f"workload {w.name}", flush=True)
    k, v = W.fill_tokens(w)
    c = _fill(w, dev, rot, k, v)
    assert c.offset == w.T and c.capacity == O.required_capacity(0, 0, w.T)
    q = W.queries(w)
    out = c.attend(q.to(dev), scale=1 / 16, causal=True)
    out_nc = c.attend(q.to(dev), scale=1 / 16, causal=False)
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.Hkv):
            ref = _check_slab(c, k, v, b, h, blocks, w.dtype)
            _check_attention(c, q, out, b, h, ref, blocks, True, w.name)
            _check_attention(c, q, out_nc, b, h, ref, blocks, False, w.name)


@pytest.mark.parametrize("cid", [3, 5])
def test_large_workloads_every_slab(cid, dev, rot, blocks):
    """Full-size cache: every (b, kv head) slab checked whole against the
    oracle (packed words, scales and biases bit for bit; the attention of its
    query rows within the tolerance), attention in the automatic launch
    configuration."""
    w = W.WORKLOADS[cid]
    print(f"workload {w.name}: generating inputs", flush=True)
    k, v = W.fill_tokens(w)
    c = _fill(w, dev, rot, k, v)
    q = W.queries(w)
    out = c.attend(q.to(dev), scale=1 / 16, causal=True)
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.Hkv):
            print(f"  slab b={b} h={h}", flush=True)
            ref = _check_slab(c, k, v, b, h, blocks, w.dtype)
            _check_attention(c, q, out, b, h, ref, blocks, True, w.name)


def test_append_verify_trim_reattend(dev, rot, blocks):
    """Fill 8192, append 2048 prefill tokens, append the 4-token verify block
    and attend it with the causal mask at the offset, trim the last 2 and
    re-attend the 2 surviving rows, then append one token (overwriting the
    stale row) and decode."""
    w = W.WORKLOADS[4]
    k0, v0 = W.fill_tokens(w)
    k1, v1 = W.append_tokens(w)
    k2, v2 = W.verify_tokens(w)
    q = W.queries(w, L=w.verify)
    c = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
    oc = O.QuantKVCache(dtype=w.dtype)
    caps = []
    for kk, vv in ((k0, v0), (k1, v1), (k2, v2)):
        c.append(kk.to(dev), vv.to(dev))
        oc.append(kk.float().numpy(), vv.float().numpy(), blocks)
        caps.append((c.capacity, c.offset))
        assert (c.capacity, c.offset) == (oc.capacity, oc.offset)
    assert caps == [(8192, 8192), (10240, 10240), (10496, 10244)]
    out = c.attend(q.to(dev), scale=1 / 16, causal=True)
    torch.cuda.synchronize()
    got = R.device_rows(c, 0, 0)
    for b in range(w.B):
        for h in range(w.Hkv):
            got = R.device_rows(c, b, h)
            ref = {n: oc.arrays[n][b, h, :oc.offset] for _, n in R.NAMES}
            R.assert_slab_equal(got, ref, f"b={b} h={h}")
    ref_out = O.attention(q.float().numpy(), oc, 1 / 16, True, blocks)
    assert float(np.abs(out.cpu().numpy() - ref_out).max()) <= ATOL

    # commit 2 of the 4 verified tokens: trim the rejected 2, re-attend rows 0-1
    assert c.commit_verified(4, 2) == 2 and oc.trim(2) == 2
    assert c.offset == oc.offset == 10242
    q2 = q[:, :, :2].contiguous()
    out2 = c.attend(q2.to(dev), scale=1 / 16, causal=True)
    torch.cuda.synchronize()
    ref2 = O.attention(q2.float().numpy(), oc, 1 / 16, True, blocks)
    assert float(np.abs(out2.cpu().numpy() - ref2).max()) <= ATOL
    # the surviving rows see exactly the keys they saw in the verify block
    assert float(np.abs(out2.cpu().numpy() - out[:, :, :2].cpu().numpy()).max()) <= 1e-5

    # one more token overwrites the stale row 10242; decode over 10243 keys
    k3, v3 = k2[:, :, 3:4].contiguous(), v2[:, :, 3:4].contiguous()
    c.append(k3.to(dev), v3.to(dev))
    oc.append(k3.float().numpy(), v3.float().numpy(), blocks)
    q3 = W.queries(w, L=1, stream=W.STREAM_VERIFY)
    out3 = c.attend(q3.to(dev), scale=1 / 16, causal=True)
    torch.cuda.synchronize()
    for b in range(w.B):
        for h in range(w.Hkv):
            got = R.device_rows(c, b, h, rows=np.arange(10240, 10243))
            ref = {n: oc.arrays[n][b, h, 10240:10243] for _, n in R.NAMES}
            R.assert_slab_equal(got, ref, f"after re-append b={b} h={h}")
    ref3 = O.attention(q3.float().numpy(), oc, 1 / 16, True, blocks)
    assert float(np.abs(out3.cpu().numpy() - ref3).max()) <= ATOL


# ------------------------------------------------------------ edge cases --

CASES = [
    # B, Hq, Hkv, T, L, dtype, dist
    (1, 1, 1, 1, 1, "bf16", "normal"),
    (2, 4, 2, 63, 3, "bf16", "normal"),
    (1, 6, 2, 65, 1, "f16", "student_t3"),
    (3, 2, 2, 300, 4, "bf16", "uniform"),
    (1, 16, 2, 1000, 4, "bf16", "normal"),     # 32 rows per kv head
    (1, 32, 2, 777, 4, "f16", "normal"),       # 64 rows per kv head
    (2, 8, 1, 4097, 2, "bf16", "student_t3"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_T{}_L{}_{}_{}".format(*c))
@pytest.mark.parametrize("use_rot", [True, False])
def test_ragged_shapes(case, use_rot, dev, rot, blocks):
    B, Hq, Hkv, T, L, dtype, dist = case
    bl = blocks if use_rot else None
    k = W.random_rows([T, 1], (B, Hkv, T, 256), dtype, dist)
    v = W.random_rows([T, 2], (B, Hkv, T, 256), dtype, dist)
    q = W.random_rows([T, 3], (B, Hq, L, 256), dtype, dist)
    c = rbq.RotatedQuantKVCache(B, Hkv, dtype=W._TORCH_DTYPES[dtype], device=dev,
                                rot=rot if use_rot else None)
    c.append(k.to(dev), v.to(dev))
    outs = {causal: c.attend(q.to(dev), scale=1 / 16, causal=causal) for causal in (True, False)}
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(Hkv):
            ref = _check_slab(c, k, v, b, h, bl, dtype)
            for causal, out in outs.items():
                _check_attention(c, q, out, b, h, ref, bl, causal, str(case))


@pytest.mark.parametrize("splits", [1, 2, 7, 64, 512])
def test_split_count_independence(splits, dev, rot, blocks):
    B, Hq, Hkv, T, L = 2, 8, 2, 3000, 2
    k = W.random_rows([5, 1], (B, Hkv, T, 256), "bf16")
    v = W.random_rows([5, 2], (B, Hkv, T, 256), "bf16")
    q = W.random_rows([5, 3], (B, Hq, L, 256), "bf16")
    c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
    c.append(k.to(dev), v.to(dev))
    base = c.attend(q.to(dev), scale=1 / 16, splits=1)
    out = c.attend(q.to(dev), scale=1 / 16, splits=splits)
    again = c.attend(q.to(dev), scale=1 / 16, splits=splits)
    torch.cuda.synchronize()
    assert float((out - base).abs().max()) <= 1e-5
    assert torch.equal(out, again)  # deterministic
    ref = R.oracle_rows(k[0, 1].float().numpy(), v[0, 1].float().numpy(), blocks, "bf16")
    _check_attention(c, q, out, 0, 1, ref, blocks, True, f"splits={splits}")


def test_chunked_appends_equal_one_shot(dev, rot):
    """Appending rows in chunks (with growth in between) gives the same bits
    as one append (row independence of the quantizer)."""
    B, Hkv, T = 2, 2, 700
    k = W.random_rows([6, 1], (B, Hkv, T, 256), "bf16", "student_t3")
    v = W.random_rows([6, 2], (B, Hkv, T, 256), "bf16")
    a = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
    a.append(k.to(dev), v.to(dev))
    b = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
    for s, e in ((0, 1), (1, 255), (255, 256), (256, 513), (513, 700)):
        b.append(k[:, :, s:e].contiguous().to(dev), v[:, :, s:e].contiguous().to(dev))
    torch.cuda.synchronize()
    assert a.offset == b.offset == T
    for name in a.arrays:
        assert torch.equal(a.rows()[name], b.rows()[name]), name


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_long_ragged_append_bit_exact(dtype, dev, rot, blocks):
    """A long append (4102 rows: a ragged last workgroup) equals the oracle bit
    for bit and equals the same rows appended in two chunks."""
    B, Hkv, T = 1, 2, 2051
    print(f"[long append] {dtype} rows={B * Hkv * T}", flush=True)
    tdt = W._TORCH_DTYPES[dtype]
    k = W.random_rows([8, 1], (B, Hkv, T, 256), dtype, "student_t3")
    v = W.random_rows([8, 2], (B, Hkv, T, 256), dtype)
    a = rbq.RotatedQuantKVCache(B, Hkv, dtype=tdt, device=dev, rot=rot)
    a.append(k.to(dev), v.to(dev))
    b = rbq.RotatedQuantKVCache(B, Hkv, dtype=tdt, device=dev, rot=rot)
    for s0, e0 in ((0, 1000), (1000, T)):
        b.append(k[:, :, s0:e0].contiguous().to(dev), v[:, :, s0:e0].contiguous().to(dev))
    torch.cuda.synchronize()
    for name in a.arrays:
        assert torch.equal(a.rows()[name], b.rows()[name]), name
    for h in range(Hkv):
        ref = R.oracle_rows(k[0, h].float().numpy(), v[0, h].float().numpy(), blocks, dtype)
        R.assert_slab_equal(R.device_rows(a, 0, h), ref, f"slab h={h}")


def test_trim_then_append_equals_fresh_cache(dev, rot):
    B, Hkv, T = 1, 2, 300
    k = W.random_rows([7, 1], (B, Hkv, T, 256), "bf16")
    v = W.random_rows([7, 2], (B, Hkv, T, 256), "bf16")
    kx = W.random_rows([7, 3], (B, Hkv, 5, 256), "bf16")
    a = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
    a.append(k.to(dev), v.to(dev))
    a.append(kx.to(dev), kx.to(dev))
    assert a.trim(5) == 5
    a.append(k[:, :, :3].contiguous().to(dev), v[:, :, :3].contiguous().to(dev))
    fresh = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
    fresh.append(torch.cat([k, k[:, :, :3]], 2).to(dev), torch.cat([v, v[:, :, :3]], 2).to(dev))
    torch.cuda.synchronize()
    assert a.offset == fresh.offset == T + 3
    for name in a.arrays:
        assert torch.equal(a.rows()[name], fresh.rows()[name]), name


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_quantizer_special_groups_without_rotation(dtype, dev):
    """Exact grid groups, round-half-even ties and constant groups, fed
    unrotated so the quantizer sees them as they are."""
    rows = []
    for levels in (16, 8):
        rows.append([-2.0 + (j % levels) / 4.0 for j in range(256)])
    g = [5.0] * 64
    g[0], g[1], g[2:6] = 0.0, 15.0, [0.5, 1.5, 2.5, 3.5]
    rows.append(g * 4)
    rows.append([1.375] * 64 + [0.0] * 64 + [-3.0] * 64 + list(np.linspace(-1, 1, 64)))
    x = torch.tensor(rows, dtype=torch.float32).to(W._TORCH_DTYPES[dtype])
    x = x.reshape(1, 1, len(rows), 256)
    c = rbq.RotatedQuantKVCache(1, 1, dtype=W._TORCH_DTYPES[dtype], device=dev, rot=None)
    c.append(x.to(dev), x.to(dev))
    torch.cuda.synchronize()
    ref = R.oracle_rows(x[0, 0].float().numpy(), x[0, 0].float().numpy(), None, dtype)
    R.assert_slab_equal(R.device_rows(c, 0, 0), ref, "special groups")


def test_error_statuses_through_the_binding(dev, rot):
    c = rbq.RotatedQuantKVCache(1, 2, device=dev, rot=rot)
    k = W.random_rows(8, (1, 2, 300, 256), "bf16").to(dev)
    c.append(k, k)
    q = W.random_rows(9, (1, 4, 1, 256), "bf16").to(dev)
    with pytest.raises(capi.RbqError) as e:
        c.attend(W.random_rows(9, (1, 3, 1, 256), "bf16").to(dev))
    assert e.value.status == capi.RBQ_EINVAL
    with pytest.raises(capi.RbqError) as e:
        c.attend(W.random_rows(9, (1, 4, 301, 256), "bf16").to(dev))
    assert e.value.status == capi.RBQ_ERANGE
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    need = capi.rbq_quant_attn_workspace_bytes(c.desc, 4, 1, 4)
    assert need > 0
    with pytest.raises(capi.RbqError) as e:
        capi.rbq_quant_attn_decode(c.desc, q, 1 / 16, True, rot, out, splits=4, ws=None)
    assert e.value.status == capi.RBQ_EWORKSPACE
    small = torch.zeros(need - 1, dtype=torch.uint8, device=dev)
    with pytest.raises(capi.RbqError) as e:
        capi.rbq_quant_attn_decode(c.desc, q, 1 / 16, True, rot, out, splits=4, ws=small)
    assert e.value.status == capi.RBQ_EWORKSPACE
    # appending beyond capacity through the raw call writes nothing
    off = c.offset
    with pytest.raises(capi.RbqError) as e:
        big = W.random_rows(10, (1, 2, c.capacity, 256), "bf16").to(dev)
        capi.rbq_kv_quant_append(c.desc, big, big, rot)
    assert e.value.status == capi.RBQ_ECAPACITY and c.offset == off
    torch.cuda.synchronize()

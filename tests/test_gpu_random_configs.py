"""GPU parity over seeded random configurations, through the whole path:
head_dim, group size, K and V widths, dtype, rotation form and precision,
batch, heads, cache length (appended in one to three chunks), query rows,
key splits and mask type drawn at random; the packed cache bit for bit
against the oracle and the attention within 2e-3 of it.  The draws reach
every attention kernel (the dedicated 8-row blocks, the tile kernel's
single-wave, paired-row, register-staged and four-wave shapes, the prefill
kernel) with shapes no hand-written case picked; a few draws are steered
to 96 or more rows per kv head, 4-bit K and groups of 64 or 128 so that the
prefill kernel takes them (bf16 or fp16, any head_dim).  Also
seeded random sequences of cache operations (appends, trims, attention
calls, one-call decoding steps, snapshots and restores), the cache compared
with the oracle's after every operation.
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
BITS = (2, 3, 4, 5, 6, 8)


def _draw(i):
    """Configuration i: (D, group, kbits, vbits, dtype, two_sided, round_rot,
    B, Hkv, n_rep, T, chunks, L, splits, mask)."""
    rng = np.random.default_rng([2026, i])
    prefill = i % 8 == 7
    D = int(rng.choice([64, 128, 256]))
    groups = [g for g in (32, 64, 128) if g <= D]
    gs = int(rng.choice(groups)) if not prefill else int(rng.choice([g for g in (64, 128) if g <= D]))
    kb = int(rng.choice(BITS)) if not prefill else 4
    vb = int(rng.choice(BITS)) if not prefill else int(rng.choice([2, 3, 4]))
    if not prefill and rng.random() < 0.3:
        D, gs, kb, vb = 256, 64, 4, 3  # the default layout now and then
    dtype = str(rng.choice(["bf16", "f16"]))
    two = bool(rng.random() < 0.4)
    rr = bool(rng.random() < 0.25)
    B = int(rng.integers(1, 3))
    Hkv = int(rng.choice([1, 2, 4]))
    n_rep = int(rng.choice([1, 2, 4, 8])) if not prefill else 8
    T = int(rng.integers(40, 700))
    n_chunks = int(rng.integers(1, 4))
    cuts = sorted(int(x) for x in rng.integers(1, T, size=n_chunks - 1))
    L = int(rng.integers(1, min(T, 24) + 1)) if not prefill else int(rng.integers(12, min(T, 40) + 1))
    splits = int(rng.choice([0, 0, 1, 3]))
    mask = str(rng.choice(["none", "none", "bool", "add"]))
    return (D, gs, kb, vb, dtype, two, rr, B, Hkv, n_rep, T, tuple(cuts), L, splits, mask)


CONFIGS = [(i, _draw(i)) for i in range(96)]


def _cid(ic):
    i, (D, gs, kb, vb, dtype, two, rr, B, Hkv, n_rep, T, cuts, L, splits, mask) = ic
    return (f"{i:02d}_D{D}_g{gs}_k{kb}v{vb}_{dtype}{'_2s' if two else ''}{'_rr' if rr else ''}"
            f"_B{B}_H{Hkv * n_rep}-{Hkv}_T{T}_L{L}_s{splits}_{mask}")


@pytest.fixture(scope="module")
def dev():
    return torch.device("cuda:0")


@pytest.mark.parametrize("cfg", CONFIGS, ids=_cid)
def test_random_configuration(cfg, dev):
    i, (D, gs, kb, vb, dtype, two, rr, B, Hkv, n_rep, T, cuts, L, splits, mask) = cfg
    print(f"[random config] {_cid(cfg)}", flush=True)
    seed = 7000 + i
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
    edges = [0, *cuts, T]
    for a, b in zip(edges[:-1], edges[1:]):
        if b > a:
            c.append(k[:, :, a:b].contiguous().to(dev), v[:, :, a:b].contiguous().to(dev))
            oc.append(k[:, :, a:b].float().numpy(), v[:, :, a:b].float().numpy(), blocks)
    torch.cuda.synchronize()
    rows = c.rows()
    for name, oname in NAMES:
        got = rows[name].cpu()
        got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
        ref = oc.arrays[oname][:, :, :oc.offset]
        assert got.shape == ref.shape, name
        assert np.array_equal(got, ref), f"{name}: {int((got != ref).sum())} mismatches"

    Hq = Hkv * n_rep
    q = W.random_rows([seed, 3], (B, Hq, L, D), dtype)
    rng = np.random.default_rng([seed, 4])
    m_np = m_dev = None
    if mask == "bool":
        m_np = rng.random(size=(B, Hq, L, T)) < 0.5
        m_np[0, Hq - 1, L - 1, :] = False  # a row that keeps no key
        m_dev = torch.from_numpy(m_np).to(dev)
    elif mask == "add":
        m_np = rng.normal(0.0, 2.0, size=(B, Hq, L, T)).astype(np.float32)
        m_dev = torch.from_numpy(m_np).to(dev)
    scale = D ** -0.5
    out = c.attend(q.to(dev), scale=scale, causal=True, splits=splits, mask=m_dev)
    torch.cuda.synchronize()
    ref = O.attention(q.float().numpy(), oc, scale, True, blocks, mask=m_np)
    err = float(np.abs(out.cpu().numpy() - ref).max())
    assert err <= ATOL, err


def _assert_same_cache(c, oc, what):
    assert c.offset == oc.offset, (what, c.offset, oc.offset)
    if oc.offset == 0:
        return
    rows = c.rows()
    for name, oname in NAMES:
        got = rows[name].cpu()
        got = got.numpy().view(np.uint32) if "words" in name else got.float().numpy()
        ref = oc.arrays[oname][:, :, :oc.offset]
        assert np.array_equal(got, ref), f"{what}, {name}: {int((got != ref).sum())} mismatches"


# random sequences of cache operations on a random configuration: appends of
# 1-200 rows, trims, attention calls, one-call decoding steps (append n rows
# and attend with L = n rows, causal at the new offset), snapshots and
# restores; the cache against the oracle's after every operation
@pytest.mark.parametrize("seed", range(24))
def test_random_operation_sequence(seed, dev):
    rng = np.random.default_rng([2027, seed])
    D = int(rng.choice([64, 128, 256]))
    gs = int(rng.choice([g for g in (32, 64, 128) if g <= D]))
    kb, vb = int(rng.choice(BITS)), int(rng.choice(BITS))
    if rng.random() < 0.4:
        D, gs, kb, vb = 256, 64, 4, 3
    dtype = str(rng.choice(["bf16", "f16"]))
    two = bool(rng.random() < 0.4)
    B, Hkv = int(rng.integers(1, 3)), int(rng.choice([1, 2]))
    Hq = Hkv * int(rng.choice([1, 2, 8]))
    print(f"[random operations] seed {seed}: D{D} g{gs} k{kb}v{vb} {dtype} B{B} H{Hq}-{Hkv}",
          flush=True)
    tdt = W._TORCH_DTYPES[dtype]
    blocks = O.rotation_blocks(W.rotation_draws(seed, D), mode="two_sided" if two else "printed")
    rot = rbq.build_block_so4(D, seed, dev, two_sided=two)
    c = rbq.RotatedQuantKVCache(B, Hkv, dtype=tdt, device=dev, rot=rot, head_dim=D,
                                group_size=gs, k_bits=kb, v_bits=vb)
    oc = O.QuantKVCache(k_bits=kb, v_bits=vb, dtype=dtype, group=gs)
    snap = None
    for step in range(10):
        op = str(rng.choice(["append", "append", "trim", "attend", "step", "snapshot", "restore"]))
        if c.offset == 0 and op in ("attend", "trim", "snapshot"):
            op = "append"
        what = f"step {step} {op}"
        if op in ("append", "step"):
            n = int(rng.integers(1, 201)) if op == "append" else int(rng.integers(1, 5))
            k = W.random_rows([seed, step, 1], (B, Hkv, n, D), dtype, "student_t3")
            v = W.random_rows([seed, step, 2], (B, Hkv, n, D), dtype)
            if op == "append":
                c.append(k.to(dev), v.to(dev))
                oc.append(k.float().numpy(), v.float().numpy(), blocks)
            else:
                q = W.random_rows([seed, step, 3], (B, Hq, n, D), dtype)
                out = c.append_attend(k.to(dev), v.to(dev), q.to(dev), scale=D ** -0.5, causal=True)
                torch.cuda.synchronize()
                oc.append(k.float().numpy(), v.float().numpy(), blocks)
                ref = O.attention(q.float().numpy(), oc, D ** -0.5, True, blocks)
                err = float(np.abs(out.cpu().numpy() - ref).max())
                assert err <= ATOL, (what, err)
        elif op == "trim":
            n = int(rng.integers(0, c.offset + 1))
            assert c.trim(n) == oc.trim(n)
        elif op == "attend":
            L = int(rng.integers(1, min(c.offset, 16) + 1))
            splits = int(rng.choice([0, 1, 3]))
            q = W.random_rows([seed, step, 4], (B, Hq, L, D), dtype)
            out = c.attend(q.to(dev), scale=D ** -0.5, causal=True, splits=splits)
            torch.cuda.synchronize()
            ref = O.attention(q.float().numpy(), oc, D ** -0.5, True, blocks)
            err = float(np.abs(out.cpu().numpy() - ref).max())
            assert err <= ATOL, (what, err)
        elif op == "snapshot":
            snap = (c.snapshot(), O.snapshot([oc]))
        elif op == "restore" and snap is not None:
            c.restore(snap[0])
            O.restore([oc], snap[1])
        torch.cuda.synchronize()
        _assert_same_cache(c, oc, what)

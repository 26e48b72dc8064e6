"""Benchmark of the quantized-KV decode step on one MI355X.

One step is one decode step of the whole path on the batched-decode workload
(B=8, 16 q heads / 2 kv heads, head_dim 256, T=32768 cached tokens, bf16,
group 64, K 4-bit / V 3-bit): the current token's K/V rows are rotated,
quantized, packed and appended at row T-1 (so attention sees T tokens), the
fused attention of the rotated query over the packed cache runs with the
causal mask at the offset and the inverse rotation of its output, and the
token is trimmed again so every step sees the same T.  The append and the
attention are one library call (``rbq_kv_append_attn_decode``: the attention
kernel writes the token's rows itself); the same step as two calls is timed
beside it.  The rotation blocks are built once before timing.  The step's
launches are issued from Python (``--graph`` replays them from a captured HIP
graph instead).

Inputs are synthetic (``workloads``), resident in HBM before timing.  The
cache is replicated (default 4 copies, 512 MiB) and the steps cycle through
the copies so that the 256 MB Infinity Cache cannot serve the 128 MiB a step
reads.

Prints ONE JSON line: ``value`` = effective HBM GB/s of the step (algorithmic
bytes / step time), plus tokens/s, the roofline of the attention kernel
(HIP events around back-to-back launches of it on the stream it runs on) and
the CPU oracle timed on a bounded sample of the same work.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ATTN_SRC = os.path.join(ROOT, "rotated_bit_quantized_amd", "csrc", "rbq_attn_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_batched_decode.json")


def algorithmic_bytes(w, T: int) -> dict:
    """Bytes one step must move at minimum.  Per cached token per kv head:
    K 32 words (128 B) + 4 bf16 scales + 4 bf16 biases, V 24 words (96 B) +
    4 + 4 bf16 = 256 B.  Plus q (bf16) in and the fp32 output, and for the
    appended token 2 x 512 B of bf16 K/V read and 256 B written."""
    cache = w.B * w.Hkv * T * 256
    q = w.B * w.Hq * w.L * w.D * 2
    out = w.B * w.Hq * w.L * w.D * 4
    append = w.B * w.Hkv * 1 * (2 * w.D * 2 + 256)
    return {"attn": cache + q + out, "append": append, "step": cache + q + out + append}


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(per_launch_alg: float):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != source_hash(ATTN_SRC):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, seconds: float = 12.0) -> dict:
    """The oracle (as it is) on one (batch, kv head) slab of the same workload,
    repeated for about ``seconds``: dequantise the slab's T packed K/V rows and
    attend its query rows over them, one thread.  The oracle's own packed
    rows of the slab are built first (not timed)."""
    from threadpoolctl import threadpool_limits

    import workloads as W
    from oracle import rbq_oracle as O

    blocks = O.rotation_blocks(W.rotation_draws(W.ROTATION_SEED, w.D))
    q = W.queries(w).float().numpy()
    n_rep = w.Hq // w.Hkv
    # slab (b=0, kv head 0) of the workload's fill, quantized by the oracle (not timed)
    rk = np.random.default_rng([w.cid, W.STREAM_K])
    rv = np.random.default_rng([w.cid, W.STREAM_V])
    k = W.to_dtype(rk.standard_normal((w.T, w.D)), w.dtype).float().numpy()
    v = W.to_dtype(rv.standard_normal((w.T, w.D)), w.dtype).float().numpy()
    kw, ks, kb = O.quantize_rows(k, blocks, 4, w.dtype)
    vw, vs, vb = O.quantize_rows(v, blocks, 3, w.dtype)
    done_slabs, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        while elapsed < seconds:
            t0 = time.perf_counter()
            khat = O.dequantize(O.unpack(kw, 4, w.D), ks, kb)
            vhat = O.dequantize(O.unpack(vw, 3, w.D), vs, vb)
            for r in range(n_rep):
                O.attention_row(q[0, r, 0], khat, vhat, w.T, 1 / 16, blocks)
            elapsed += time.perf_counter() - t0
            done_slabs += 1
    per_slab_bytes = w.T * 256 + n_rep * w.D * (2 + 4)
    return {
        "value": round(done_slabs * per_slab_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done_slabs} passes over one (batch, kv head) slab: dequantise "
                  f"{w.T} packed K/V rows and attend {n_rep} query rows, numpy fp64, "
                  f"1 thread, {elapsed:.1f} s",
        "tokens_per_s": round(done_slabs / (w.B * w.Hkv) * w.B / elapsed, 4),
    }


def tree_verify(rbq, W, dev, rot, n_calls: int = 200) -> dict:
    """Batched verification of P draft paths: a batch-1 cache of 10240 tokens
    (the append_verify fill + append) tiled over P = 4 paths, 4 draft tokens
    appended per path, then the fused attention of all paths' draft rows
    (16 q heads / 2 kv heads) under a boolean tree mask (every draft token sees
    the prefix and its ancestors: token 2 and 3 both follow token 1).  16 cache
    replicas (21 MB each, 336 MB in all) so that the Infinity Cache cannot
    serve a call.  Reports the masked call, the same call with the causal mask
    instead, and the tile copy (1 -> 4 paths)."""
    P, Hkv, Hq, T0, L = 4, 2, 16, 10240, 4
    k = W.random_rows([40, 1], (1, Hkv, T0, 256), "bf16").to(dev)
    v = W.random_rows([40, 2], (1, Hkv, T0, 256), "bf16").to(dev)
    one = rbq.RotatedQuantKVCache(1, Hkv, device=dev, rot=rot)
    one.append(k, v)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # tile copy, timed on its own (one batch-1 cache into 4 paths, repeatedly)
    tiled = []
    for _ in range(16):
        c = rbq.RotatedQuantKVCache(1, Hkv, device=dev, rot=rot)
        c.arrays = {n: a.clone() for n, a in one.arrays.items()}
        c.desc = rbq.rbq_kv_cache.from_buffer_copy(one.desc)
        c._bind(c.desc, c.arrays, one.capacity)
        tiled.append(c)
    dsts = []
    for c in tiled[:2]:
        d = rbq.RotatedQuantKVCache(1, Hkv, device=dev, rot=rot)
        d.desc = rbq.rbq_kv_cache.from_buffer_copy(one.desc)
        d.desc.B = P
        d.arrays = one._alloc(one.capacity, P)
        d._bind(d.desc, d.arrays, one.capacity)
        dsts.append(d)
    for i in range(4):
        rbq.rbq_kv_copy_batch(tiled[i % 16].desc, 0, 0, dsts[i % 2].desc)
    ev0.record(stream)
    for i in range(40):
        rbq.rbq_kv_copy_batch(tiled[i % 16].desc, 0, 0, dsts[i % 2].desc)
    ev1.record(stream)
    torch.cuda.synchronize()
    tile_us = ev0.elapsed_time(ev1) * 1e3 / 40
    tile_bytes = Hkv * T0 * 256 * (1 + P)
    del dsts
    kd = W.random_rows([41, 1], (P, Hkv, L, 256), "bf16").to(dev)
    vd = W.random_rows([41, 2], (P, Hkv, L, 256), "bf16").to(dev)
    for c in tiled:
        c.tile(P)
        c.append(kd, vd)
    T = T0 + L
    parent = [-1, 0, 1, 1]
    keep = torch.zeros(L, T, dtype=torch.bool)
    keep[:, :T0] = True
    for i in range(L):
        j = i
        while j >= 0:
            keep[i, T0 + j] = True
            j = parent[j]
    keep = keep.to(dev)
    q = W.random_rows([41, 3], (P, Hq, L, 256), "bf16").to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = tiled[0].workspace(Hq, L)

    def timed(mask, causal):
        for i in range(50):
            c = tiled[i % 16]
            rbq.rbq_quant_attn_decode(c.desc, q, 1 / 16, causal, rot, out, 0, ws, mask)
        ev0.record(stream)
        for i in range(n_calls):
            c = tiled[i % 16]
            rbq.rbq_quant_attn_decode(c.desc, q, 1 / 16, causal, rot, out, 0, ws, mask)
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / n_calls

    masked_us = timed(keep, False)
    causal_us = timed(None, True)
    alg = P * Hkv * T * 256 + P * Hq * L * 256 * (2 + 4) + L * T
    gbs = alg / (masked_us * 1e-6) / 1e9
    return {
        "what": f"{P} draft paths x {L} tokens over {T0} cached tokens, {Hq}/{Hkv} heads, "
                "bf16, boolean tree mask (rbq_quant_attn_decode_mask); 16 cache replicas",
        "bound": "hbm",
        "alg_bytes_per_call": alg,
        "avg_us": round(masked_us, 3),
        "achieved": round(gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "verified_tokens_per_s": round(P * L / (masked_us * 1e-6), 1),
        "causal_mask_avg_us": round(causal_us, 3),
        "tile_copy": {"avg_us": round(tile_us, 3), "bytes": tile_bytes,
                      "achieved": round(tile_bytes / (tile_us * 1e-6) / 1e9, 2)},
    }


def long_context(rbq, W, dev, rot, n_calls: int = 300) -> dict:
    """Decode over the long-context workload: B=1, 16 q heads / 2 kv heads,
    head_dim 256, T=262144, bf16, Student-t (nu = 3) K, K4/V3 group 64: the
    key range of each kv head split 128 ways and merged by log-sum-exp.  Four
    cache replicas (512 MiB) cycled against the Infinity Cache; HIP events
    around back-to-back calls (after 600 warm-up calls).  Bytes: as the
    batched decode, 256 per token and kv head plus q and out."""
    w = W.WORKLOADS[5]
    k, v = W.fill_tokens(w)
    base = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
    base.append(k.to(dev), v.to(dev))
    del k, v
    caches = [base]
    for _ in range(3):
        c = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
        c.arrays = {n: a.clone() for n, a in base.arrays.items()}
        c.desc = rbq.capi.rbq_kv_cache.from_buffer_copy(base.desc)
        c._bind(c.desc, c.arrays, base.capacity)
        caches.append(c)
    q = W.queries(w).to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = base.workspace(w.Hq, w.L)
    S = rbq.capi.rbq_quant_attn_splits(base.desc, w.Hq, w.L)
    stream = torch.cuda.current_stream()
    for i in range(600):
        rbq.capi.rbq_quant_attn_decode(caches[i % 4].desc, q, 1 / 16, True, rot, out, 0, ws)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(n_calls):
        rbq.capi.rbq_quant_attn_decode(caches[i % 4].desc, q, 1 / 16, True, rot, out, 0, ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / n_calls
    alg = w.B * w.Hkv * w.T * 256 + w.B * w.Hq * w.D * (2 + 4)
    gbs = alg / (us * 1e-6) / 1e9
    return {
        "what": f"decode, B=1, {w.Hq}/{w.Hkv} heads, head_dim 256, T={w.T}, bf16, Student-t K, "
                f"K4/V3 group 64, {S} key splits per kv head",
        "bound": "hbm",
        "alg_bytes_per_call": alg,
        "avg_us": round(us, 3),
        "achieved": round(gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(w.B / (us * 1e-6), 1),
    }


def append_throughput(rbq, W, dev, rot, n_calls: int = 32) -> dict:
    """The append (a2 + a3) of a prefill chunk on the append+verify shapes:
    B=4, 16 q heads / 2 kv heads, head_dim 256, bf16, K4/V3 group 64, 2048
    new tokens after 8192 cached; 16 input sets (268 MB) and 4 caches cycled
    so that the Infinity Cache cannot serve the inputs; append then trim,
    HIP events around the back-to-back appends.  Bytes: the bf16 K and V
    rows read plus the packed rows written."""
    B, Hkv, T0, n, D = 4, 2, 8192, 2048, 256
    k = W.random_rows([70, 1], (B, Hkv, T0, D), "bf16").to(dev)
    v = W.random_rows([70, 2], (B, Hkv, T0, D), "bf16").to(dev)
    caches = []
    for _ in range(4):
        c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot)
        c.append(k, v)
        c.reserve(n)
        caches.append(c)
    del k, v
    base = W.random_rows([70, 3], (B, Hkv, n, D), "bf16").to(dev)
    ins = [(base.roll(i, dims=3).contiguous(), base.roll(-i, dims=3).contiguous()) for i in range(16)]
    stream = torch.cuda.current_stream()
    for i in range(8):
        c = caches[i % 4]
        rbq.rbq_kv_quant_append(c.desc, ins[i % 16][0], ins[i % 16][1], rot)
        rbq.rbq_kv_trim(c.desc, n)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(n_calls):
        c = caches[i % 4]
        rbq.rbq_kv_quant_append(c.desc, ins[i % 16][0], ins[i % 16][1], rot)
        rbq.rbq_kv_trim(c.desc, n)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / n_calls
    rows = B * Hkv * n
    nbytes = rows * (2 * D * 2 + 256)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {
        "what": f"append of {n} tokens after {T0} cached, B={B}, {Hkv} kv heads, head_dim 256, bf16, "
                "K4/V3 group 64 (rbq_kv_quant_append: rotate, quantize, pack, write)",
        "bound": "alu",
        "note": "VALU-bound, not HBM-bound: about 470 vector instructions per row and wave "
                "(fp64 rotation, group min/max, codes, packing); frac is against the HBM peak, "
                "for context",
        "bytes_per_call": nbytes,
        "avg_us": round(us, 3),
        "achieved": round(gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(B * n / (us * 1e-6), 1),
    }


def prefill(rbq, W, dev, rot, n_calls: int = 10, head_dim: int = 256) -> dict:
    """Prefill-length attention over the quantized cache: B=1, 16 q heads /
    2 kv heads, head_dim 256, bf16, K4/V3 group 64; a cache of 8192 tokens,
    a chunk of L = 2048 new tokens appended (rotated, quantized, packed), then
    the fused attention of the chunk's 2048 query rows per head over the
    10240 cached tokens with the causal mask at the offset (the dedicated
    kernel's 8-row blocks).  With ``head_dim=128`` the cache is head_dim 128,
    group 64, K4/V4, two-sided rotation (the tile kernel's 64-row blocks).
    Algorithmic flops: 4 * head_dim per (query row, visible key) (q.k and
    p.v, multiply-add = 2)."""
    Hkv, Hq, T0, L = 2, 16, 8192, 2048
    D = head_dim
    if D != 256:
        rot = rbq.build_block_so4(D, 0, dev, two_sided=True)
    cfg = {} if D == 256 else dict(head_dim=D, group_size=64, k_bits=4, v_bits=4)
    k = W.random_rows([50, 1], (1, Hkv, T0, D), "bf16").to(dev)
    v = W.random_rows([50, 2], (1, Hkv, T0, D), "bf16").to(dev)
    kn = W.random_rows([50, 3], (1, Hkv, L, D), "bf16").to(dev)
    vn = W.random_rows([50, 4], (1, Hkv, L, D), "bf16").to(dev)
    q = W.random_rows([50, 5], (1, Hq, L, D), "bf16").to(dev)
    c = rbq.RotatedQuantKVCache(1, Hkv, device=dev, rot=rot, **cfg)
    c.append(k, v)
    c.reserve(L)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the chunk's append, timed on its own (append then trim, repeatedly)
    for _ in range(3):
        c.append(kn, vn)
        c.trim(L)
    ev0.record(stream)
    for _ in range(n_calls):
        c.append(kn, vn)
        c.trim(L)
    ev1.record(stream)
    torch.cuda.synchronize()
    append_us = ev0.elapsed_time(ev1) * 1e3 / n_calls
    c.append(kn, vn)
    T = T0 + L
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = c.workspace(Hq, L)
    for _ in range(2):
        rbq.rbq_quant_attn_decode(c.desc, q, D ** -0.5, True, rot, out, 0, ws)
    ev0.record(stream)
    for _ in range(n_calls):
        rbq.rbq_quant_attn_decode(c.desc, q, D ** -0.5, True, rot, out, 0, ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / n_calls
    pairs = Hq * (L * (T - L) + L * (L + 1) // 2)  # (query row, visible key) pairs
    flops = 4 * D * pairs
    tfs = flops / (us * 1e-6) / 1e12
    return {
        "what": (f"prefill chunk: {L} new tokens over {T0} cached (T={T}), B=1, {Hq}/{Hkv} heads, "
                 "head_dim 256, bf16, K4/V3 group 64, causal at the offset (the dedicated kernel: "
                 "4096 blocks of 8 query rows)") if D == 256 else
                (f"prefill chunk: {L} new tokens over {T0} cached (T={T}), B=1, {Hq}/{Hkv} heads, "
                 "head_dim 128, bf16, K4/V4 group 64, two-sided rotation, causal at the offset "
                 "(the tile kernel: 512 blocks of 64 query rows)"),
        "bound": "mfma",
        "alg_flops_per_call": flops,
        "avg_us": round(us, 2),
        "achieved": round(tfs, 2),
        "peak": 2500.0,
        "unit": "TFLOP/s",
        "frac": round(tfs / 2500.0, 4),
        "note": "fp16 MFMA issued per algorithmic flop: 2 (query and probability operands "
                "split hi + lo); the dense fp16 peak is the reference",
        "tokens_per_s": round(L / (us * 1e-6), 1),
        "append_chunk_us": round(append_us, 2),
    }


def variant_decode(rbq, W, dev, n_calls: int = 200) -> dict:
    """Decode over a cache of another configuration (the general kernels):
    B=8, 16 q heads / 2 kv heads, head_dim 128, group 64, K 4-bit / V 4-bit,
    two-sided rotation, T=32768, bf16; 5 cache replicas (about 380 MB) cycled
    so that the Infinity Cache cannot serve a call."""
    B, Hkv, Hq, T, D, gs, kb, vb = 8, 2, 16, 32768, 128, 64, 4, 4
    rot = rbq.build_block_so4(D, 0, dev, two_sided=True)
    k = W.random_rows([60, 1], (B, Hkv, T, D), "bf16").to(dev)
    v = W.random_rows([60, 2], (B, Hkv, T, D), "bf16").to(dev)
    caches = []
    for _ in range(5):
        c = rbq.RotatedQuantKVCache(B, Hkv, device=dev, rot=rot, head_dim=D, group_size=gs,
                                    k_bits=kb, v_bits=vb)
        c.append(k, v)
        caches.append(c)
    del k, v
    q = W.random_rows([60, 3], (B, Hq, 1, D), "bf16").to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    ws = caches[0].workspace(Hq, 1)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(20):
        rbq.rbq_quant_attn_decode(caches[i % 5].desc, q, D ** -0.5, True, rot, out, 0, ws)
    ev0.record(stream)
    for i in range(n_calls):
        rbq.rbq_quant_attn_decode(caches[i % 5].desc, q, D ** -0.5, True, rot, out, 0, ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / n_calls
    row = D * kb // 8 + D * vb // 8 + 4 * (D // gs) * 2  # packed K, V and the four meta arrays
    alg = B * Hkv * T * row + B * Hq * D * (2 + 4)
    gbs = alg / (us * 1e-6) / 1e9
    return {
        "what": f"decode, B={B}, {Hq}/{Hkv} heads, head_dim {D}, group {gs}, K{kb}/V{vb}, "
                f"two-sided rotation, T={T}, bf16 (tile kernel)",
        "bound": "hbm",
        "alg_bytes_per_call": alg,
        "avg_us": round(us, 3),
        "achieved": round(gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(B / (us * 1e-6), 1),
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000,
                    help="untimed steps first: the GPU clock takes about 100 ms of work to settle")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--splits", type=int, default=0, help="key splits (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph (on this stack a replay "
                         "costs more than the two launches it holds)")
    ap.add_argument("--leg", choices=["prefill", "variant_decode", "variant_prefill", "tree_verify",
                                      "append", "long_context"],
                    help="run only this secondary measurement and print its object "
                         "(for profiling it on its own; not the benchmark line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        return 2

    import rotated_bit_quantized_amd as rbq
    from rotated_bit_quantized_amd import capi
    import workloads as W

    if args.leg is not None:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        rot = rbq.build_block_so4(256, W.ROTATION_SEED, dev)
        leg = {"prefill": lambda: prefill(rbq, W, dev, rot),
               "variant_decode": lambda: variant_decode(rbq, W, dev),
               "variant_prefill": lambda: prefill(rbq, W, dev, rot, head_dim=128),
               "tree_verify": lambda: tree_verify(rbq, W, dev, rot),
               "append": lambda: append_throughput(rbq, W, dev, rot),
               "long_context": lambda: long_context(rbq, W, dev, rot)}[args.leg]
        print(json.dumps({args.leg: leg()}), flush=True)
        return 0

    w = W.WORKLOADS[3]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rot = rbq.build_block_so4(w.D, W.ROTATION_SEED, dev)

    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    k, v = W.fill_tokens(w)
    q = W.queries(w).to(dev)
    k_new = k[:, :, w.T - 1:].contiguous().to(dev)
    v_new = v[:, :, w.T - 1:].contiguous().to(dev)
    base = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
    base.append(k[:, :, :w.T - 1].contiguous().to(dev), v[:, :, :w.T - 1].contiguous().to(dev))
    del k, v
    caches = [base]
    for _ in range(args.replicas - 1):
        c = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
        c.arrays = {n: a.clone() for n, a in base.arrays.items()}
        c.desc = capi.rbq_kv_cache.from_buffer_copy(base.desc)
        c._bind(c.desc, c.arrays, base.capacity)
        caches.append(c)
    assert base.capacity >= w.T
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    after = capi.rbq_kv_cache.from_buffer_copy(base.desc)
    after.offset = w.T  # the attention runs over T rows
    nb_ws = capi.rbq_quant_attn_workspace_bytes(after, w.Hq, w.L, args.splits)
    ws = torch.empty(nb_ws, dtype=torch.uint8, device=dev) if nb_ws else None
    splits_used = capi.rbq_quant_attn_splits(after, w.Hq, w.L) if args.splits == 0 \
        else args.splits
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    # One step: the token's rows appended at row T-1 and the attention over T
    # rows in one library call (the attention kernel writes the rows itself),
    # then the trim back to T-1 (host-side bookkeeping).  `step_two_calls` is
    # the same step as the append call followed by the attention call.
    def step(i):
        c = caches[i % len(caches)]
        capi.rbq_kv_append_attn_decode(c.desc, k_new, v_new, q, 1 / 16, True, rot, out,
                                       args.splits, ws)
        capi.rbq_kv_trim(c.desc, 1)

    def step_two_calls(i):
        c = caches[i % len(caches)]
        capi.rbq_kv_quant_append(c.desc, k_new, v_new, rot)
        capi.rbq_quant_attn_decode(c.desc, q, 1 / 16, True, rot, out, args.splits, ws)
        capi.rbq_kv_trim(c.desc, 1)

    # --graph: one HIP graph per cache replica holds the step's launches with
    # their arguments as captured; the trim back to T-1 is host-side
    # bookkeeping only.
    graphs = []
    if args.graph:
        cap = torch.cuda.Stream()
        for c in caches:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                capi.rbq_kv_append_attn_decode(c.desc, k_new, v_new, q, 1 / 16, True, rot, out,
                                               args.splits, ws)
            capi.rbq_kv_trim(c.desc, 1)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step(i)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    # the same number of steps as two calls (append, then attention)
    for i in range(min(args.warmup, 200)):
        step_two_calls(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_two_calls(i)
    torch.cuda.synchronize()
    total_two = time.perf_counter() - t0

    # The attention kernel alone: back-to-back launches on the stream it runs
    # on, HIP events at both ends (an event pair around every launch would add
    # the dispatch gap it forces to each measurement).
    n_attn = max(100, args.steps // 2)
    for c in caches:  # T rows, as in the step
        capi.rbq_kv_quant_append(c.desc, k_new, v_new, rot)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(n_attn):
        c = caches[i % len(caches)]
        capi.rbq_quant_attn_decode(c.desc, q, 1 / 16, True, rot, out, args.splits, ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    attn_us = ev0.elapsed_time(ev1) * 1e3 / n_attn
    for c in caches:
        capi.rbq_kv_trim(c.desc, 1)

    # Cache snapshot (the prefix copy of the six arrays, rows [0, T)): copies
    # from the rotating replicas into two alternating snapshot buffer sets, so
    # that neither side is served by the Infinity Cache; HIP events around
    # back-to-back copies on the stream.
    snaps = [base.snapshot(), base.snapshot()]
    n_copy = 40
    for i in range(4):
        capi.rbq_kv_copy_prefix(caches[i % len(caches)].desc, snaps[i % 2].desc)
    ev0.record(stream)
    for i in range(n_copy):
        capi.rbq_kv_copy_prefix(caches[i % len(caches)].desc, snaps[i % 2].desc)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy_us = ev0.elapsed_time(ev1) * 1e3 / n_copy
    copy_bytes = 2 * w.B * w.Hkv * (w.T - 1) * 256  # read + write of the prefix
    copy_gbs = copy_bytes / (copy_us * 1e-6) / 1e9
    del snaps

    print("[bench] tree verification", file=sys.stderr, flush=True)
    tree = tree_verify(rbq, W, dev, rot)
    print("[bench] prefill chunk", file=sys.stderr, flush=True)
    pre = prefill(rbq, W, dev, rot)
    print("[bench] append of a prefill chunk", file=sys.stderr, flush=True)
    app = append_throughput(rbq, W, dev, rot)
    print("[bench] long context", file=sys.stderr, flush=True)
    lng = long_context(rbq, W, dev, rot)
    print("[bench] decode and prefill, head_dim 128 K4/V4", file=sys.stderr, flush=True)
    var = variant_decode(rbq, W, dev)
    pre128 = prefill(rbq, W, dev, rot, head_dim=128)

    nbytes = algorithmic_bytes(w, w.T)
    ms_per_step = total * 1e3 / args.steps
    value = nbytes["step"] / (ms_per_step * 1e-3) / 1e9
    attn_avg_s = attn_us * 1e-6
    achieved = nbytes["attn"] / attn_avg_s / 1e9
    traffic = measured_traffic(nbytes["attn"])

    result = {
        "metric": "quantized-KV decode attention: effective HBM GB/s (% of peak) and tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={w.B}, {w.Hq} q heads / {w.Hkv} kv heads, head_dim {w.D}, "
                        f"T={w.T} cached tokens, L={w.L}, bf16 N(0,1), group 64, K4/V3, "
                        f"rotation seed 0",
            "B": w.B, "H_q": w.Hq, "H_kv": w.Hkv, "head_dim": w.D, "T": w.T, "L": w.L,
            "splits": splits_used, "cache_replicas": len(caches),
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.B * w.L / (ms_per_step * 1e-3), 1),
        "step_bytes": nbytes["step"],
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "attn_mfma_kernel (rbq_quant_attn_decode): HIP events around "
                      f"{n_attn} back-to-back launches on its stream",
            "alg_bytes_per_launch": nbytes["attn"],
            "avg_launch_us": round(attn_avg_s * 1e6, 3),
        },
        "step": ("HIP graph replay" if graphs else "eager launches") +
                " of rbq_kv_append_attn_decode (append of the token and attention in one call)",
        "two_call_step": {
            "what": "the same step as rbq_kv_quant_append + rbq_quant_attn_decode (eager)",
            "ms_per_step": round(total_two * 1e3 / args.steps, 5),
            "value": round(nbytes["step"] / (total_two / args.steps) / 1e9, 2),
        },
        "snapshot": {
            "what": f"cache snapshot: prefix copy of the six arrays, {w.T - 1} rows x "
                    f"{w.B * w.Hkv} (b, kv head) slabs (rbq_kv_copy_prefix, copy_prefix_kernel)",
            "bound": "hbm",
            "bytes_per_copy": copy_bytes,
            "avg_us": round(copy_us, 3),
            "achieved": round(copy_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(copy_gbs / HBM_PEAK_GBS, 4),
        },
        "tree_verify": tree,
        "prefill": pre,
        "variant_decode": var,
        "variant_prefill": pre128,
        "append": app,
        "long_context": lng,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

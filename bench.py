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
beside it.  The rotation blocks are built once before timing.

Inputs are synthetic (``workloads``), resident in HBM before timing.  Caches
are replicated and the steps cycle through the copies so that the 256 MB
Infinity Cache cannot serve the bytes a step reads.

Every timed object states how many untimed calls ran before its timing and
gives the median, 10th and 90th percentile over windows of back-to-back
calls (HIP events on the stream the calls run on).  The GPU clock is settled
first by a fixed number of untimed steps.

Prints ONE JSON line: ``value`` = effective HBM GB/s of the step (algorithmic
bytes / step time) over exactly ``--steps`` timed steps after ``--warmup``
untimed ones, plus tokens/s, the roofline of the attention kernel, one object
per workload (tiny, decode_gqa, batched_decode, append_verify,
long_context) with the CPU oracle's time for the same work, the plain
streaming-read rate of the GPU, and the secondary measurements.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ATTN_SRC = os.path.join(ROOT, "rotated_bit_quantized_amd", "csrc", "rbq_attn_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_batched_decode.json")
APPEND_ALU_FILE = os.path.join(ROOT, "profiles", "append_prefill_chunk_alu.json")
# vector lane operations per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
# (a wave64 instruction holds its SIMD 4 cycles; x 2 flops per FMA gives the
# 78.6 TFLOP/s fp64 and unpacked fp32 vector peak)
VALU_PEAK_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12
PROBE_LIB = os.path.join(ROOT, "rotated_bit_quantized_amd", "librbq_probe.so")
SETTLE_CALLS = 3000   # untimed steps that bring the GPU clock to its steady state first


def algorithmic_bytes(w, T: int, n_new: int = 1, L: int = None) -> dict:
    """Bytes one step must move at minimum.  Per cached token per kv head:
    K 32 words (128 B) + 4 bf16 scales + 4 bf16 biases, V 24 words (96 B) +
    4 + 4 bf16 = 256 B.  Plus q (dtype) in and the fp32 output, and for the
    n_new appended tokens 2 x 512 B of K/V read and 256 B written."""
    L = w.L if L is None else L
    cache = w.B * w.Hkv * T * 256
    q = w.B * w.Hq * L * w.D * 2
    out = w.B * w.Hq * L * w.D * 4
    append = w.B * w.Hkv * n_new * (2 * w.D * 2 + 256)
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


def append_issue_cycles():
    """VALU issue cycles per appended row from the committed counter summary
    of the append kernel, if it was taken on the current kernel sources."""
    try:
        with open(APPEND_ALU_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    now = [source_hash(os.path.join(ROOT, p)) for p in t.get("kernel_sources", [])]
    if not now or now != t.get("kernel_sources_sha256_16"):
        return None
    return t.get("valu_issue_cycles_per_row")


def timed_windows(fn, untimed: int, n_windows: int, per_window: int) -> dict:
    """``untimed`` calls of fn(i), then ``n_windows`` windows of ``per_window``
    back-to-back calls, each bracketed by HIP events on the current stream;
    microseconds per call: median, 10th and 90th percentile over the windows."""
    stream = torch.cuda.current_stream()
    for i in range(untimed):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    vals = []
    i0 = untimed
    for _ in range(n_windows):
        e0.record(stream)
        for i in range(per_window):
            fn(i0 + i)
        e1.record(stream)
        torch.cuda.synchronize()
        vals.append(e0.elapsed_time(e1) * 1e3 / per_window)
        i0 += per_window
    return {"median": round(statistics.median(vals), 3),
            "p10": round(float(np.percentile(vals, 10)), 3),
            "p90": round(float(np.percentile(vals, 90)), 3),
            "mean": round(statistics.fmean(vals), 3),
            "untimed_calls": untimed, "windows": n_windows, "calls_per_window": per_window}


def graph_windows(fn, steps_per_graph: int, untimed: int, n_windows: int) -> dict:
    """Latency-bound steps: ``steps_per_graph`` consecutive calls of fn(i)
    captured in one HIP graph; ``untimed`` replays first, then one replay per
    window (HIP events around it); microseconds per step."""
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        for i in range(steps_per_graph):
            fn(i)
    torch.cuda.synchronize()
    for _ in range(untimed):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    vals = []
    for _ in range(n_windows):
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        vals.append(e0.elapsed_time(e1) * 1e3 / steps_per_graph)
    return {"median": round(statistics.median(vals), 3),
            "p10": round(float(np.percentile(vals, 10)), 3),
            "p90": round(float(np.percentile(vals, 90)), 3),
            "untimed_calls": untimed * steps_per_graph, "windows": n_windows,
            "calls_per_window": steps_per_graph,
            "launch": f"HIP graph of {steps_per_graph} steps, one replay per window"}


def replicas(rbq, capi, base, n: int) -> list:
    """``base`` and n - 1 device copies of its six arrays (same descriptor)."""
    out = [base]
    for _ in range(n - 1):
        c = rbq.RotatedQuantKVCache(base.desc.B, base.desc.H_kv, dtype=base.dtype,
                                    device=base.device, rot=base.rot)
        c.arrays = {k: a.clone() for k, a in base.arrays.items()}
        c.desc = capi.rbq_kv_cache.from_buffer_copy(base.desc)
        c._bind(c.desc, c.arrays, base.capacity)
        out.append(c)
    return out


def stream_read_probe(dev) -> dict:
    """The practical HBM read ceiling of this GPU: a plain streaming read
    (``librbq_probe.so``) of 128 MiB (the size the batched decode reads per
    call) from 4 rotating buffers, and of 2 GiB, with the non-temporal hint;
    the best of a few launch shapes."""
    lib = ctypes.CDLL(PROBE_LIB)
    f = lib.rbq_probe_stream_read
    f.restype = ctypes.c_int32
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32, ctypes.c_void_p]
    sink = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    res = {}
    for size, nbuf, label in ((134217728, 4, "128MiB"), (2147483648, 1, "2GiB")):
        bufs = [torch.ones(size // 4, dtype=torch.int32, device=dev) for _ in range(nbuf)]
        best = None
        for blocks, unroll in ((256, 8), (2048, 1), (512, 4)):
            st = torch.cuda.current_stream().cuda_stream

            def call(i, blocks=blocks, unroll=unroll):
                rc = f(bufs[i % nbuf].data_ptr(), size, sink.data_ptr(), blocks, unroll, 1, st)
                assert rc == 0
            t = timed_windows(call, 8, 5, 20 if size < 1e9 else 4)
            gbs = size / (t["median"] * 1e-6) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks, unroll, t)
        res[label] = {"GBps": round(best[0], 1), "pct_of_hbm_peak": round(100 * best[0] / HBM_PEAK_GBS, 2),
                      "us": best[3]["median"], "launch": f"{best[1]} workgroups x 256 threads, "
                      f"{best[2]} 16-byte loads in flight per thread"}
        del bufs
    res["what"] = ("plain streaming read (rbq_probe_stream_read, non-temporal 16-byte loads): the "
                   "achievable HBM read rate on this GPU, context for the kernels' fractions of the "
                   "8 TB/s peak")
    return res


# ---------------------------------------------------------------- oracle --

def oracle_time(W, O, w, T_sample: int, rows, n_keys_of, scale_to: float, what: str) -> dict:
    """The oracle as it stands, one thread, on a bounded sample of a
    workload's attention: one (batch, kv head) slab of ``T_sample`` rows of
    the workload's fill (quantized and packed by the oracle first, not
    timed), then ``attention_row`` (dequantise the slab, scores, softmax,
    values, inverse rotation) for ``rows`` query rows.  The time is scaled by
    ``scale_to`` to the whole step."""
    from threadpoolctl import threadpool_limits

    blocks = O.rotation_blocks(W.rotation_draws(W.ROTATION_SEED, w.D))
    k, v = W.keys_values(dataclasses_replace(w, B=1, Hkv=1), [w.cid, W.STREAM_K],
                         [w.cid, W.STREAM_V], T_sample)
    oc = O.QuantKVCache(dtype=w.dtype)
    oc.append(k.float().numpy(), v.float().numpy(), blocks)
    q = W.queries(w, L=max(1, w.L)).float().numpy()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        khat, vhat = oc.dequant_kv(0, 0)
        for (h, i) in rows:
            O.attention_row(q[0, h % w.Hq, i % q.shape[2]], khat, vhat, n_keys_of(i), 1 / 16, blocks)
        el = time.perf_counter() - t0
    return {"s_per_step": round(el * scale_to, 4), "cores": 1, "kind": "oracle",
            "sample": f"{what}: {el:.2f} s for one slab of {T_sample} rows and {len(rows)} query "
                      f"rows, scaled x{scale_to:g}"}


def dataclasses_replace(w, **kw):
    import dataclasses
    return dataclasses.replace(w, **kw)


# ---------------------------------------------------------- per workload --

def decode_workload(rbq, capi, W, O, dev, rot, cid: int, n_rep_caches: int, use_graph: bool,
                    oracle: bool) -> dict:
    """One decode step of a workload (tiny, decode_gqa, long_context): the
    token's rows appended at row T-1 and the attention over T rows in one
    call (``rbq_kv_append_attn_decode``), then the trim back to T-1.  Also the
    attention call alone over T rows."""
    w = W.WORKLOADS[cid]
    k, v = W.fill_tokens(w)
    q = W.queries(w).to(dev)
    kn = k[:, :, w.T - 1:].contiguous().to(dev)
    vn = v[:, :, w.T - 1:].contiguous().to(dev)
    base = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
    base.append(k[:, :, :w.T - 1].contiguous().to(dev), v[:, :, :w.T - 1].contiguous().to(dev))
    del k, v
    caches = replicas(rbq, capi, base, n_rep_caches)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    after = capi.rbq_kv_cache.from_buffer_copy(base.desc)
    after.offset = w.T
    nb = capi.rbq_quant_attn_workspace_bytes(after, w.Hq, w.L, 0)
    ws = torch.zeros(nb, dtype=torch.uint8, device=dev) if nb else None
    S = capi.rbq_quant_attn_splits(after, w.Hq, w.L)

    def step(i):
        c = caches[i % len(caches)]
        capi.rbq_kv_append_attn_decode(c.desc, kn, vn, q, 1 / 16, True, rot, out, 0, ws)
        capi.rbq_kv_trim(c.desc, 1)

    if use_graph:
        for i in range(SETTLE_CALLS // 3):
            step(i)
        t = graph_windows(step, 100, 10, 10)
    else:
        t = timed_windows(step, SETTLE_CALLS // 3, 10, 100)
    for c in caches:
        capi.rbq_kv_quant_append(c.desc, kn, vn, rot)

    def attn(i):
        capi.rbq_quant_attn_decode(caches[i % len(caches)].desc, q, 1 / 16, True, rot, out, 0, ws)

    ta = graph_windows(attn, 100, 10, 10) if use_graph else timed_windows(attn, 200, 10, 100)
    nbytes = algorithmic_bytes(w, w.T)
    us = t["median"]
    gbs = nbytes["step"] / (us * 1e-6) / 1e9
    res = {
        "workload": f"{w.name}: B={w.B}, {w.Hq} q heads / {w.Hkv} kv heads, head_dim {w.D}, "
                    f"T={w.T}, L={w.L}, {w.dtype}, K {w.k_dist}, group 64, K4/V3",
        "step": "rbq_kv_append_attn_decode (the token's append and the attention in one call) + trim",
        "key_splits": S, "cache_replicas": len(caches),
        "us_per_step": t,
        "bytes_per_step": nbytes["step"],
        "GBps": round(gbs, 1),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.B * w.L / (us * 1e-6), 1),
        "attention_call_us": ta,
        "attention_GBps": round(nbytes["attn"] / (ta["median"] * 1e-6) / 1e9, 1),
    }
    if oracle:
        T_s = min(w.T, 32768)
        slabs = w.B * w.Hkv
        res["oracle"] = oracle_time(W, O, w, T_s, [(h, 0) for h in range(w.n_rep)],
                                    lambda i: T_s, slabs * w.T / T_s,
                                    f"{w.n_rep} query rows of one slab")
        res["oracle"]["gpu_speedup"] = round(res["oracle"]["s_per_step"] / (us * 1e-6), 1)
    return res


def append_verify_workload(rbq, capi, W, O, dev, rot, oracle: bool) -> dict:
    """The append+verify workload: a cache filled with 8192 tokens and a
    2048-token prefill chunk appended (timed on its own), then the step: the
    4-token verify block appended and attended with the causal mask at the
    offset (``rbq_kv_append_attn_decode`` with n = L = 4), trimmed back.  Also
    the re-attend after trimming 2 of the 4 (L = 2 over 10242 keys).  16
    cache replicas (21 MB each) against the Infinity Cache."""
    w = W.WORKLOADS[4]
    k0, v0 = W.fill_tokens(w)
    k1, v1 = W.append_tokens(w)
    k2, v2 = W.verify_tokens(w)
    base = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
    base.append(k0.to(dev), v0.to(dev))
    k1d, v1d = k1.to(dev), v1.to(dev)
    base.reserve(w.append + w.verify)
    # the prefill chunk's append, timed on its own (append then trim)
    app_caches = replicas(rbq, capi, base, 4)

    def app(i):
        c = app_caches[i % 4]
        capi.rbq_kv_quant_append(c.desc, k1d, v1d, rot)
        capi.rbq_kv_trim(c.desc, w.append)

    t_app = timed_windows(app, 16, 5, 8)
    del app_caches
    base.append(k1d, v1d)
    caches = replicas(rbq, capi, base, 16)
    kd, vd = k2.to(dev), v2.to(dev)
    q = W.queries(w, L=w.verify).to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    after = capi.rbq_kv_cache.from_buffer_copy(base.desc)
    after.offset += w.verify
    nb = capi.rbq_quant_attn_workspace_bytes(after, w.Hq, w.verify, 0)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev)

    def step(i):
        c = caches[i % 16]
        capi.rbq_kv_append_attn_decode(c.desc, kd, vd, q, 1 / 16, True, rot, out, 0, ws)
        capi.rbq_kv_trim(c.desc, w.verify)

    t = timed_windows(step, SETTLE_CALLS // 3, 10, 100)
    # re-attend: the 2 surviving rows after trimming 2 of the 4
    for c in caches:
        capi.rbq_kv_quant_append(c.desc, kd, vd, rot)
        capi.rbq_kv_trim(c.desc, w.trim)
    q2 = q[:, :, :w.verify - w.trim].contiguous()
    out2 = torch.empty(q2.shape, dtype=torch.float32, device=dev)

    def reattend(i):
        capi.rbq_quant_attn_decode(caches[i % 16].desc, q2, 1 / 16, True, rot, out2, 0, ws)

    t_re = timed_windows(reattend, 200, 10, 100)
    T = w.T + w.append + w.verify
    nbytes = algorithmic_bytes(w, T, n_new=w.verify, L=w.verify)
    us = t["median"]
    gbs = nbytes["step"] / (us * 1e-6) / 1e9
    app_bytes = w.B * w.Hkv * w.append * (2 * w.D * 2 + 256)
    res = {
        "workload": f"{w.name}: B={w.B}, {w.Hq}/{w.Hkv} heads, head_dim 256, bf16, cache {w.T} + "
                    f"{w.append} appended, verify block of {w.verify} (T={T}), trim {w.trim}",
        "step": f"the verify block: {w.verify} rows appended and attended (L={w.verify}, causal at "
                "the offset) by rbq_kv_append_attn_decode, then trimmed",
        "cache_replicas": 16,
        "us_per_step": t,
        "bytes_per_step": nbytes["step"],
        "GBps": round(gbs, 1),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "verified_tokens_per_s": round(w.B * w.verify / (us * 1e-6), 1),
        "reattend_L2_us": t_re,
        "prefill_chunk_append": {"us": t_app, "bytes": app_bytes,
                                 "GBps": round(app_bytes / (t_app["median"] * 1e-6) / 1e9, 1),
                                 "tokens_per_s": round(w.B * w.append / (t_app["median"] * 1e-6), 1)},
    }
    if oracle:
        T_s = T
        rows = [(h, i) for h in range(w.n_rep) for i in range(w.verify)]
        res["oracle"] = oracle_time(W, O, w, T_s, rows, lambda i: T_s - w.verify + i + 1,
                                    w.B * w.Hkv, f"{len(rows)} verify rows of one slab")
        res["oracle"]["gpu_speedup"] = round(res["oracle"]["s_per_step"] / (us * 1e-6), 1)
    return res


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
    tile_t = timed_windows(lambda i: rbq.rbq_kv_copy_batch(tiled[i % 16].desc, 0, 0, dsts[i % 2].desc),
                           untimed=4, n_windows=5, per_window=20)
    tile_us = tile_t["mean"]
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
        return timed_windows(
            lambda i: rbq.rbq_quant_attn_decode(tiled[i % 16].desc, q, 1 / 16, causal, rot, out, 0,
                                                ws, mask),
            untimed=50, n_windows=10, per_window=n_calls // 4)

    masked_t = timed(keep, False)
    causal_t = timed(None, True)
    masked_us, causal_us = masked_t["mean"], causal_t["mean"]
    alg = P * Hkv * T * 256 + P * Hq * L * 256 * (2 + 4) + L * T
    gbs = alg / (masked_us * 1e-6) / 1e9
    return {
        "what": f"{P} draft paths x {L} tokens over {T0} cached tokens, {Hq}/{Hkv} heads, "
                "bf16, boolean tree mask (rbq_quant_attn_decode_mask); 16 cache replicas",
        "bound": "hbm",
        "alg_bytes_per_call": alg,
        "avg_us": round(masked_us, 3),
        "us": masked_t,
        "achieved": round(gbs, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "verified_tokens_per_s": round(P * L / (masked_us * 1e-6), 1),
        "causal_mask_avg_us": round(causal_us, 3),
        "causal_mask_us": causal_t,
        "tile_copy": {"avg_us": round(tile_us, 3), "us": tile_t, "bytes": tile_bytes,
                      "achieved": round(tile_bytes / (tile_us * 1e-6) / 1e9, 2)},
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
    def one(i):
        c = caches[i % 4]
        rbq.rbq_kv_quant_append(c.desc, ins[i % 16][0], ins[i % 16][1], rot)
        rbq.rbq_kv_trim(c.desc, n)

    t = timed_windows(one, untimed=8, n_windows=5, per_window=n_calls)
    us = t["mean"]
    rows = B * Hkv * n
    nbytes = rows * (2 * D * 2 + 256)
    gbs = nbytes / (us * 1e-6) / 1e9
    cyc = append_issue_cycles()
    alu = None
    if cyc is not None:
        # lane operations the call's vector instructions occupy (issue cycles
        # x 16 lanes) per second, against the chip's lane-operation rate
        tl = rows * cyc * 16 / (us * 1e-6) / 1e12
        alu = {"bound": "alu", "achieved": round(tl, 2), "peak": round(VALU_PEAK_TLANEOPS, 2),
               "unit": "T VALU lane-op/s", "frac": round(tl / VALU_PEAK_TLANEOPS, 4),
               "issue_cycles_per_row": cyc,
               "from": "profiles/append_prefill_chunk_alu.json (rocprofv3 SQ counters)"}
    return {
        "what": f"append of {n} tokens after {T0} cached, B={B}, {Hkv} kv heads, head_dim 256, bf16, "
                "K4/V3 group 64 (rbq_kv_quant_append: rotate, quantize, pack, write)",
        "bound": "alu",
        "note": "bound by vector issue, not HBM: 422 vector instructions per row and wave "
                "(fp64 rotation, group min/max, codes, packing); `roofline` is against the "
                "vector lane-operation peak (null when the kernel sources changed since the "
                "counters were taken), achieved / peak / frac against the HBM peak, for context",
        "roofline": alu,
        "bytes_per_call": nbytes,
        "avg_us": round(us, 3),
        "us": t,
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
    10240 cached tokens with the causal mask at the offset (the prefill
    kernel's 128-row blocks).  With ``head_dim=128`` the cache is head_dim 128,
    group 64, K4/V4, two-sided rotation (the same kernel's head_dim-128 build).
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
    t = timed_windows(lambda i: rbq.rbq_quant_attn_decode(c.desc, q, D ** -0.5, True, rot, out, 0, ws),
                      untimed=2, n_windows=5, per_window=n_calls // 5)
    us = t["mean"]
    pairs = Hq * (L * (T - L) + L * (L + 1) // 2)  # (query row, visible key) pairs
    flops = 4 * D * pairs
    tfs = flops / (us * 1e-6) / 1e12
    return {
        "what": (f"prefill chunk: {L} new tokens over {T0} cached (T={T}), B=1, {Hq}/{Hkv} heads, "
                 "head_dim 256, bf16, K4/V3 group 64, causal at the offset (the prefill kernel: "
                 "256 blocks of 128 query rows)") if D == 256 else
                (f"prefill chunk: {L} new tokens over {T0} cached (T={T}), B=1, {Hq}/{Hkv} heads, "
                 "head_dim 128, bf16, K4/V4 group 64, two-sided rotation, causal at the offset "
                 "(the prefill kernel: 256 blocks of 128 query rows)"),
        "bound": "mfma",
        "alg_flops_per_call": flops,
        "avg_us": round(us, 2),
        "us": t,
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
    t = timed_windows(
        lambda i: rbq.rbq_quant_attn_decode(caches[i % 5].desc, q, D ** -0.5, True, rot, out, 0, ws),
        untimed=20, n_windows=10, per_window=n_calls // 4)
    us = t["mean"]
    row = D * kb // 8 + D * vb // 8 + 4 * (D // gs) * 2  # packed K, V and the four meta arrays
    alg = B * Hkv * T * row + B * Hq * D * (2 + 4)
    gbs = alg / (us * 1e-6) / 1e9
    return {
        "what": f"decode, B={B}, {Hq}/{Hkv} heads, head_dim {D}, group {gs}, K{kb}/V{vb}, "
                f"two-sided rotation, T={T}, bf16 (tile kernel)",
        "bound": "hbm",
        "alg_bytes_per_call": alg,
        "avg_us": round(us, 3),
        "us": t,
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
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps right before the timed ones (after the clock-settling "
                         f"phase of {SETTLE_CALLS} untimed steps)")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--splits", type=int, default=0, help="key splits (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true",
                    help="the batched-decode step and its roofline only (for profiling)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured HIP graph (on this stack a replay "
                         "costs more than the launch it holds)")
    ap.add_argument("--leg", choices=["prefill", "variant_decode", "variant_prefill", "tree_verify",
                                      "append", "tiny", "decode_gqa", "append_verify",
                                      "long_context", "stream"],
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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rot = rbq.build_block_so4(256, W.ROTATION_SEED, dev)
    O = None
    if not args.no_cpu_baseline and args.leg is None and not args.quick:
        from oracle import rbq_oracle as O  # the CPU oracle, for the cpu_baseline figures only

    legs = {"prefill": lambda: prefill(rbq, W, dev, rot),
            "variant_decode": lambda: variant_decode(rbq, W, dev),
            "variant_prefill": lambda: prefill(rbq, W, dev, rot, head_dim=128),
            "tree_verify": lambda: tree_verify(rbq, W, dev, rot),
            "append": lambda: append_throughput(rbq, W, dev, rot),
            "tiny": lambda: decode_workload(rbq, capi, W, O, dev, rot, 1, 4, True, O is not None),
            "decode_gqa": lambda: decode_workload(rbq, capi, W, O, dev, rot, 2, 16, True,
                                                  O is not None),
            "append_verify": lambda: append_verify_workload(rbq, capi, W, O, dev, rot, O is not None),
            "long_context": lambda: decode_workload(rbq, capi, W, O, dev, rot, 5, 4, False,
                                                    O is not None),
            "stream": lambda: stream_read_probe(dev)}
    if args.leg is not None:
        print(json.dumps({args.leg: legs[args.leg]()}), flush=True)
        return 0

    w = W.WORKLOADS[3]
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    k, v = W.fill_tokens(w)
    q = W.queries(w).to(dev)
    k_new = k[:, :, w.T - 1:].contiguous().to(dev)
    v_new = v[:, :, w.T - 1:].contiguous().to(dev)
    base = rbq.RotatedQuantKVCache(w.B, w.Hkv, dtype=w.torch_dtype, device=dev, rot=rot)
    base.append(k[:, :, :w.T - 1].contiguous().to(dev), v[:, :, :w.T - 1].contiguous().to(dev))
    del k, v
    caches = replicas(rbq, capi, base, args.replicas)
    assert base.capacity >= w.T
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    after = capi.rbq_kv_cache.from_buffer_copy(base.desc)
    after.offset = w.T  # the attention runs over T rows
    nb_ws = capi.rbq_quant_attn_workspace_bytes(after, w.Hq, w.L, args.splits)
    ws = torch.zeros(nb_ws, dtype=torch.uint8, device=dev) if nb_ws else None
    splits_used = capi.rbq_quant_attn_splits(after, w.Hq, w.L) if args.splits == 0 \
        else args.splits
    torch.cuda.synchronize()

    # One step: the token's rows appended at row T-1 and the attention over T
    # rows in one library call (the attention kernel writes the rows itself),
    # then the trim back to T-1 (host-side bookkeeping).  `step_two_calls` is
    # the same step as the append call followed by the attention call.
    # the step's library call with its arguments marshalled once (a serving
    # loop repeats the same call); the work on the GPU is that of the call
    step_call = capi.prepare_append_attn_decode(caches[0].desc, k_new, v_new, q, 1 / 16, True,
                                                rot, out, args.splits, ws)

    def step(i):
        c = caches[i % len(caches)]
        step_call(c.desc)
        capi.rbq_kv_trim(c.desc, 1)

    def step_two_calls(i):
        c = caches[i % len(caches)]
        capi.rbq_kv_quant_append(c.desc, k_new, v_new, rot)
        capi.rbq_quant_attn_decode(c.desc, q, 1 / 16, True, rot, out, args.splits, ws)
        capi.rbq_kv_trim(c.desc, 1)

    # --graph: one HIP graph per cache replica holds the step's launch with
    # its arguments as captured; the trim back to T-1 is host-side only.
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

    # clock settling, then the contract: W untimed steps, K timed steps
    # bracketed by synchronisations
    for i in range(SETTLE_CALLS):
        run(i)
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(i)
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    # the step in windows (distribution), then as two calls
    step_win = timed_windows(run, 0, 10, 200)
    two_win = timed_windows(step_two_calls, 200, 10, 200)

    # The attention call alone (both kernels): back-to-back launches on the
    # stream it runs on, HIP events at both ends of each window.
    for c in caches:  # T rows, as in the step
        capi.rbq_kv_quant_append(c.desc, k_new, v_new, rot)

    def attn(i):
        capi.rbq_quant_attn_decode(caches[i % len(caches)].desc, q, 1 / 16, True, rot, out,
                                   args.splits, ws)

    attn_win = timed_windows(attn, 500, 10, 200)
    for c in caches:
        capi.rbq_kv_trim(c.desc, 1)

    nbytes = algorithmic_bytes(w, w.T)
    ms_per_step = total * 1e3 / args.steps
    value = nbytes["step"] / (ms_per_step * 1e-3) / 1e9
    attn_avg_s = attn_win["median"] * 1e-6
    achieved = nbytes["attn"] / attn_avg_s / 1e9
    traffic = measured_traffic(nbytes["attn"])
    batched = {
        "workload": f"{w.name}: B={w.B}, {w.Hq} q heads / {w.Hkv} kv heads, head_dim {w.D}, "
                    f"T={w.T}, L={w.L}, bf16 N(0,1), group 64, K4/V3",
        "step": "rbq_kv_append_attn_decode (the token's append and the attention in one call) + trim",
        "key_splits": splits_used, "cache_replicas": len(caches),
        "us_per_step": step_win,
        "bytes_per_step": nbytes["step"],
        "GBps": round(nbytes["step"] / (step_win["median"] * 1e-6) / 1e9, 1),
        "pct_of_hbm_peak": round(100 * nbytes["step"] / (step_win["median"] * 1e-6) / 1e9
                                 / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.B * w.L / (step_win["median"] * 1e-6), 1),
        "attention_call_us": attn_win,
        "attention_GBps": round(achieved, 1),
        "two_call_step_us": two_win,
    }
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
        "untimed_steps_before_timing": SETTLE_CALLS + args.warmup,
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
            "kernel": "attn_mfma_kernel + attn_mfma_merge_kernel (rbq_quant_attn_decode): median of "
                      "10 windows of 200 back-to-back calls, HIP events on their stream, after "
                      f"{SETTLE_CALLS + args.warmup + args.steps + 4700} untimed calls",
            "alg_bytes_per_launch": nbytes["attn"],
            "avg_launch_us": round(attn_avg_s * 1e6, 3),
        },
        "step": ("HIP graph replay" if graphs else "eager launches") +
                " of rbq_kv_append_attn_decode (append of the token and attention in one call)",
    }
    if args.quick:
        result["batched_decode"] = batched
        print(json.dumps(result), flush=True)
        return 0

    # Cache snapshot (the prefix copy of the six arrays, rows [0, T)): copies
    # from the rotating replicas into two alternating snapshot buffer sets, so
    # that neither side is served by the Infinity Cache.
    snaps = [base.snapshot(), base.snapshot()]

    def copy(i):
        capi.rbq_kv_copy_prefix(caches[i % len(caches)].desc, snaps[i % 2].desc)

    copy_win = timed_windows(copy, 8, 5, 20)
    copy_bytes = 2 * w.B * w.Hkv * (w.T - 1) * 256  # read + write of the prefix
    copy_gbs = copy_bytes / (copy_win["median"] * 1e-6) / 1e9
    del snaps, caches, base

    print("[bench] stream probe", file=sys.stderr, flush=True)
    stream = stream_read_probe(dev)
    per = {"tiny": None, "decode_gqa": None, "batched_decode": batched, "append_verify": None,
           "long_context": None}
    for name in ("tiny", "decode_gqa", "append_verify", "long_context"):
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        per[name] = legs[name]()
        torch.cuda.empty_cache()
    print("[bench] tree verification", file=sys.stderr, flush=True)
    tree = tree_verify(rbq, W, dev, rot)
    print("[bench] prefill chunk", file=sys.stderr, flush=True)
    pre = prefill(rbq, W, dev, rot)
    print("[bench] append of a prefill chunk", file=sys.stderr, flush=True)
    app = append_throughput(rbq, W, dev, rot)
    print("[bench] decode and prefill, head_dim 128 K4/V4", file=sys.stderr, flush=True)
    var = variant_decode(rbq, W, dev)
    pre128 = prefill(rbq, W, dev, rot, head_dim=128)

    result.update({
        "achievable_stream_read": stream,
        "workloads": per,
        "snapshot": {
            "what": f"cache snapshot: prefix copy of the six arrays, {w.T - 1} rows x "
                    f"{w.B * w.Hkv} (b, kv head) slabs (rbq_kv_copy_prefix, copy_prefix_kernel)",
            "bound": "hbm",
            "bytes_per_copy": copy_bytes,
            "us": copy_win,
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
    })
    if O is not None:
        print("[bench] timing the CPU oracle samples", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w)
        batched["oracle"] = {"s_per_step": round(w.B * w.Hkv * 256 * w.T
                                                / (result["cpu_baseline"]["value"] * 1e9), 3),
                             "cores": 1, "kind": "oracle",
                             "sample": "from cpu_baseline (one slab, scaled to the 16 slabs)"}
        batched["oracle"]["gpu_speedup"] = round(batched["oracle"]["s_per_step"]
                                                 / (step_win["median"] * 1e-6), 1)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Test-side helpers: run the CPU oracle on one (batch, kv head) slab at a time
and compare the library's device buffers with it.  Imports the oracle (tests
only) and the library binding; nothing here is imported by the product."""
from __future__ import annotations

import numpy as np
import torch

from oracle import rbq_oracle as O

CHUNK = 32768  # rows per oracle call, bounds the oracle's fp64 temporaries

NAMES = (("k_words", "kw"), ("k_scales", "ks"), ("k_biases", "kb"),
         ("v_words", "vw"), ("v_scales", "vs"), ("v_biases", "vb"))


def oracle_rows(k_rows: np.ndarray, v_rows: np.ndarray, blocks, dtype: str) -> dict:
    """Oracle quantize+pack of rows ``[n, D]`` (float32 values of the input
    dtype), in chunks.  Returns {kw, ks, kb, vw, vs, vb}."""
    parts = {n: [] for _, n in NAMES}
    for r0 in range(0, k_rows.shape[0], CHUNK):
        kw, ks, kb = O.quantize_rows(k_rows[r0:r0 + CHUNK], blocks, 4, dtype)
        vw, vs, vb = O.quantize_rows(v_rows[r0:r0 + CHUNK], blocks, 3, dtype)
        for name, val in (("kw", kw), ("ks", ks), ("kb", kb), ("vw", vw), ("vs", vs), ("vb", vb)):
            parts[name].append(val)
    return {n: np.concatenate(p) if p else None for n, p in parts.items()}


def device_rows(cache, b: int, h: int, rows=None) -> dict:
    """The library's six arrays for slab (b, h), rows [0, offset) or ``rows``
    (an index array), as numpy (words uint32, scales/biases float32)."""
    out = {}
    for name, oname in NAMES:
        a = cache.arrays[name][b, h, :cache.offset]
        if rows is not None:
            a = a[torch.as_tensor(rows, device=a.device)]
        a = a.cpu()
        out[oname] = a.numpy().view(np.uint32) if "words" in name else a.float().numpy()
    return out


def assert_slab_equal(got: dict, ref: dict, what: str = "") -> None:
    for _, n in NAMES:
        g, r = got[n], ref[n]
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)
            raise AssertionError(f"{what} {n}: {len(bad)} mismatches, first at {bad[0].tolist()} "
                                 f"got {g[tuple(bad[0])]} want {r[tuple(bad[0])]}")


def dequant_slab(ref: dict) -> tuple:
    """fp64 dequantised K and V rows of one slab from the oracle's own arrays."""
    D = ref["ks"].shape[-1] * O.GROUP
    kc = O.unpack(ref["kw"], 4, D)
    vc = O.unpack(ref["vw"], 3, D)
    return O.dequantize(kc, ref["ks"], ref["kb"]), O.dequantize(vc, ref["vs"], ref["vb"])


def oracle_attention_slab(q: np.ndarray, b: int, kvh: int, n_rep: int, khat, vhat, T: int,
                          causal: bool, blocks, scale: float) -> np.ndarray:
    """Oracle outputs ``[n_rep, L, D]`` of the q heads reading kv head ``kvh``."""
    L, D = q.shape[2], q.shape[3]
    out = np.empty((n_rep, L, D), np.float32)
    for r in range(n_rep):
        h = kvh * n_rep + r
        for i in range(L):
            n_keys = T - L + i + 1 if causal else T
            out[r, i] = O.attention_row(q[b, h, i], khat, vhat, n_keys, scale, blocks)
    return out

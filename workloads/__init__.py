"""Seeded synthetic inputs shared by the oracle, the tests, the smoke check and the bench.

This module only draws random numbers and rounds them to the input dtype.  It
holds none of the method's arithmetic (no rotation, no quantizer, no packing,
no attention), so both the CPU oracle and the HIP path can consume the same
inputs without sharing any code that decides a result.

Recipe (one generator per (config, stream), numpy PCG64):
  ``numpy.random.default_rng([config_id, stream])`` with streams
  q = 0, k = 1, v = 2, outlier channels = 3; appended tokens use
  ``[config_id, 4, 0]`` (K) and ``[config_id, 4, 1]`` (V), verify tokens
  ``[config_id, 5, 0|1]``.  Values are drawn in fp64, rounded to fp32 (RNE) and
  then to the cache dtype (RNE, by torch's conversion).

The rotation's own random numbers (the quaternion draws of the block build
on the page "quant_kv.py", section "SO(4) block rotation") are produced here
as well: for each 4-D block, four standard normals for the left quaternion,
then four for the right one, each cast to float32, from
``numpy.random.default_rng(seed)``.  The normalisation and the block product
that turn them into a rotation are method arithmetic and live on each side
separately.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

HEAD_DIM = 256
GROUP = 64
K_BITS = 4
V_BITS = 3
ROTATION_SEED = 0

STREAM_Q, STREAM_K, STREAM_V, STREAM_OUTLIER, STREAM_APPEND, STREAM_VERIFY = range(6)

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: cache shape, query block and value distribution."""

    cid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int                   # tokens in the cache when the (first) attention runs
    L: int = 1               # query rows per sequence for the timed attention
    dtype: str = "bf16"
    k_dist: str = "normal"   # "normal", "outliers" (8 channels x10 per kv head), "student_t3"
    append: int = 0          # tokens appended after the initial fill (append+verify workload)
    verify: int = 0          # verify block length (append+verify workload)
    trim: int = 0            # tokens trimmed after the verify (append+verify workload)
    D: int = HEAD_DIM

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPES[self.dtype]

    @property
    def n_rep(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    1: Workload(1, "tiny", B=1, Hq=1, Hkv=1, T=256, L=1, dtype="f16"),
    2: Workload(2, "decode_gqa", B=1, Hq=16, Hkv=2, T=4096, L=1, k_dist="outliers"),
    3: Workload(3, "batched_decode", B=8, Hq=16, Hkv=2, T=32768, L=1),
    4: Workload(4, "append_verify", B=4, Hq=16, Hkv=2, T=8192, L=4,
                append=2048, verify=4, trim=2),
    5: Workload(5, "long_context", B=1, Hq=16, Hkv=2, T=262144, L=1, k_dist="student_t3"),
}


def rotation_draws(seed: int = ROTATION_SEED, head_dim: int = HEAD_DIM) -> np.ndarray:
    """Raw quaternion draws, float32 ``[head_dim/4, 2, 4]`` (left draw, then right draw)."""
    if head_dim % 4 != 0:
        raise ValueError("head_dim must be a multiple of 4")
    rng = np.random.default_rng(seed)
    out = np.empty((head_dim // 4, 2, 4), dtype=np.float32)
    for b in range(head_dim // 4):
        out[b, 0] = rng.standard_normal(4).astype(np.float32)
        out[b, 1] = rng.standard_normal(4).astype(np.float32)
    return out


def to_dtype(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """fp64 numpy -> fp32 (RNE) -> ``dtype`` torch CPU tensor (RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return t.to(_TORCH_DTYPES[dtype])


def normal(seed, shape, dtype: str) -> torch.Tensor:
    return to_dtype(np.random.default_rng(seed).standard_normal(shape), dtype)


def outlier_channels(cid: int, Hkv: int, D: int = HEAD_DIM, n: int = 8) -> np.ndarray:
    """Per kv head, ``n`` distinct channel indices (before rotation) that get scaled x10."""
    rng = np.random.default_rng([cid, STREAM_OUTLIER])
    return np.stack([rng.choice(D, n, replace=False) for _ in range(Hkv)])


def keys_values(w: Workload, seed_k, seed_v, n: int):
    """K and V token rows ``[B, Hkv, n, D]`` of workload ``w`` in its dtype (CPU tensors)."""
    shape = (w.B, w.Hkv, n, w.D)
    rk = np.random.default_rng(seed_k)
    if w.k_dist == "student_t3":
        k64 = rk.standard_t(3, size=shape)
    else:
        k64 = rk.standard_normal(shape)
    if w.k_dist == "outliers":
        ch = outlier_channels(w.cid, w.Hkv, w.D)
        for h in range(w.Hkv):
            k64[:, h, :, ch[h]] *= 10.0
    k = to_dtype(k64, w.dtype)
    del k64
    v = normal(seed_v, shape, w.dtype)
    return k, v


def fill_tokens(w: Workload):
    """The tokens that fill the cache before the first attention: ``T`` rows each."""
    return keys_values(w, [w.cid, STREAM_K], [w.cid, STREAM_V], w.T)


def append_tokens(w: Workload):
    """Prefill tokens appended after the fill (append+verify workload)."""
    return keys_values(w, [w.cid, STREAM_APPEND, 0], [w.cid, STREAM_APPEND, 1], w.append)


def verify_tokens(w: Workload):
    """K/V rows of the verify block (append+verify workload)."""
    return keys_values(w, [w.cid, STREAM_VERIFY, 0], [w.cid, STREAM_VERIFY, 1], w.verify)


def queries(w: Workload, L: Optional[int] = None, stream: int = STREAM_Q) -> torch.Tensor:
    """Query block ``[B, Hq, L, D]`` in the workload dtype."""
    L = w.L if L is None else L
    return normal([w.cid, stream], (w.B, w.Hq, L, w.D), w.dtype)


def random_rows(seed, shape, dtype: str, dist: str = "normal", scale: float = 1.0) -> torch.Tensor:
    """Generic seeded rows for edge-case tests (any shape)."""
    rng = np.random.default_rng(seed)
    if dist == "student_t3":
        x = rng.standard_t(3, size=shape)
    elif dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape)
    else:
        x = rng.standard_normal(shape)
    return to_dtype(x * scale, dtype)

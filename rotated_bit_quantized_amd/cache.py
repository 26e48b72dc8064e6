"""Python face of the quantized KV cache: torch owns the device buffers, the
library does every step of the method.

``RotatedQuantKVCache`` follows ``AsymmetricQuantizedKVCache`` on the page
"mlx_streaming/core/cache/quant_kv.py": six arrays (K packed words, K scales,
K biases, V packed words, V scales, V biases) of shape ``[B, H_kv, capacity,
.]``, an ``offset``, growth in 256-row steps, ``trim``; plus the SO(4) block
rotation applied on append and attention and undone on the output.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import capi

HEAD_DIM = 256
GROUP = 64
K_BITS = 4
V_BITS = 3
STEP = 256


def quaternion_draws(seed: int = 0, head_dim: int = HEAD_DIM) -> np.ndarray:
    """The random numbers the block rotation draws (page quant_kv.py,
    ``build_block_so4``): numpy ``default_rng(seed)``, and for each 4-D block
    four standard normals for the left quaternion, then four for the right,
    each cast to float32.  Returns ``[head_dim/4, 2, 4]``."""
    if head_dim % 4:
        raise ValueError("head_dim must be a multiple of 4")
    rng = np.random.default_rng(seed)
    out = np.empty((head_dim // 4, 2, 4), dtype=np.float32)
    for b in range(head_dim // 4):
        out[b, 0] = rng.standard_normal(4).astype(np.float32)
        out[b, 1] = rng.standard_normal(4).astype(np.float32)
    return out


def build_block_so4(head_dim: int = HEAD_DIM, seed: int = 0, device="cuda",
                    two_sided: bool = False, round_to: Optional[torch.dtype] = None) -> torch.Tensor:
    """Rotation blocks ``float32 [head_dim/4, 4, 4]`` on ``device``
    (``build_block_so4`` without the dense matrix: only its diagonal blocks).
    ``two_sided``: the right factor is the right multiplication by conj(qR)
    that the page's ``_quat_right_conj`` docstring describes, instead of the
    printed matrix.  ``round_to``: the blocks rounded to that dtype (the
    page's ``R.astype(x.dtype)``; pair it with a cache made with
    ``round_rotated=True``)."""
    mode = capi.RBQ_ROT_TWO_SIDED if two_sided else capi.RBQ_ROT_PRINTED
    blocks = capi.rbq_rotation_build_mode(quaternion_draws(seed, head_dim), mode)
    if round_to is not None:
        if round_to not in capi.DTYPE_CODES:
            raise ValueError("round_to must be torch.float16 or torch.bfloat16")
        blocks = capi.rbq_rotation_round(blocks, capi.DTYPE_CODES[round_to])
    return torch.from_numpy(blocks).to(device)


class RotatedQuantKVCache:
    """Rotated, asymmetric quantized KV cache on one GPU (K4/V3, group 64,
    head_dim 256 by default; head_dim 64/128/256, group 32/64/128 and widths
    2/3/4/5/6/8 for K and V independently).

    ``rot`` is the device tensor of rotation blocks (or None: inputs are taken
    as already rotated and outputs stay in the rotated space, as the page's
    cache and SDPA do).  ``round_rotated``: rotated rows are rounded to the
    cache dtype (the page's own rotation precision); pass blocks rounded to
    the dtype as well (``build_block_so4(round_to=dtype)``)."""

    def __init__(self, B: int, H_kv: int, dtype: torch.dtype = torch.bfloat16,
                 device="cuda", rot: Optional[torch.Tensor] = None,
                 head_dim: int = HEAD_DIM, group_size: int = GROUP,
                 k_bits: int = K_BITS, v_bits: int = V_BITS, round_rotated: bool = False):
        if dtype not in capi.DTYPE_CODES:
            raise ValueError("dtype must be torch.float16 or torch.bfloat16")
        self.device = torch.device(device)
        self.dtype = dtype
        self.rot = rot
        self.desc = capi.rbq_kv_cache(B=B, H_kv=H_kv, head_dim=head_dim, group_size=group_size,
                                      k_bits=k_bits, v_bits=v_bits,
                                      dtype=capi.DTYPE_CODES[dtype],
                                      flags=capi.RBQ_FLAG_ROUND_ROTATED if round_rotated else 0,
                                      capacity=0, offset=0)
        self.arrays = None
        self._ws = None

    # -- page API ------------------------------------------------------------
    @property
    def offset(self) -> int:
        return int(self.desc.offset)

    @property
    def capacity(self) -> int:
        return int(self.desc.capacity)

    def empty(self) -> bool:
        return self.arrays is None

    @property
    def nbytes(self) -> int:
        """Bytes held by the six buffers (capacity rows, not offset rows)."""
        if self.arrays is None:
            return 0
        return sum(a.numel() * a.element_size() for a in self.arrays.values())

    def _alloc(self, capacity: int, B: Optional[int] = None) -> dict:
        d = self.desc
        kw = d.head_dim * d.k_bits // 32
        vw = d.head_dim * d.v_bits // 32
        ng = d.head_dim // d.group_size
        shp = (d.B if B is None else B, d.H_kv, capacity)
        return {
            "k_words": torch.empty(shp + (kw,), dtype=torch.int32, device=self.device),
            "k_scales": torch.empty(shp + (ng,), dtype=self.dtype, device=self.device),
            "k_biases": torch.empty(shp + (ng,), dtype=self.dtype, device=self.device),
            "v_words": torch.empty(shp + (vw,), dtype=torch.int32, device=self.device),
            "v_scales": torch.empty(shp + (ng,), dtype=self.dtype, device=self.device),
            "v_biases": torch.empty(shp + (ng,), dtype=self.dtype, device=self.device),
        }

    @staticmethod
    def _bind(desc: capi.rbq_kv_cache, arrays: dict, capacity: int) -> None:
        desc.capacity = capacity
        for name, t in arrays.items():
            setattr(desc, name, t.data_ptr())

    def reserve(self, n: int) -> None:
        """Grow the buffers so that n more rows fit (update_and_fetch's growth rule)."""
        cap = capi.rbq_kv_required_capacity(self.capacity, self.offset, n)
        if cap == self.capacity:
            return
        new = self._alloc(cap)
        dst = capi.rbq_kv_cache.from_buffer_copy(self.desc)
        self._bind(dst, new, cap)
        capi.rbq_kv_grow(self.desc, dst)
        self.arrays = new
        self.desc = dst

    def append(self, k: torch.Tensor, v: torch.Tensor) -> None:
        """update_and_fetch: rotate, quantize, pack and write ``k``/``v``
        ``[B, H_kv, n, head_dim]`` at ``offset``; ``offset`` advances by n."""
        n = k.shape[2]
        self.reserve(n)
        capi.rbq_kv_quant_append(self.desc, k, v, self.rot)

    update_and_fetch = append

    def trim(self, n: int) -> int:
        return capi.rbq_kv_trim(self.desc, n)

    def commit_verified(self, verified_len: int, accepted_len: int) -> int:
        return capi.rbq_kv_commit_verified(self.desc, verified_len, accepted_len)

    # -- attention -------------------------------------------------------------
    def workspace(self, H_q: int, L: int, splits: int = 0) -> Optional[torch.Tensor]:
        nb = capi.rbq_quant_attn_workspace_bytes(self.desc, H_q, L, splits)
        if nb == 0:
            return None
        if self._ws is None or self._ws.numel() < nb:
            self._ws = torch.empty(nb, dtype=torch.uint8, device=self.device)
        return self._ws

    def attend(self, q: torch.Tensor, scale: Optional[float] = None, causal: bool = True,
               splits: int = 0, out: Optional[torch.Tensor] = None,
               mask: Optional[torch.Tensor] = None) -> torch.Tensor:
        """Fused attention of ``q [B, H_q, L, head_dim]`` over rows [0, offset),
        returning float32 ``[B, H_q, L, head_dim]`` rotated back.  ``mask``
        (optional, as the page's SDPA takes an array mask): broadcastable to
        ``[B, H_q, L, keys >= offset]``, boolean (keep where true) or additive
        (float32 or the cache dtype); ``causal`` applies as well."""
        if scale is None:
            scale = self.desc.head_dim ** -0.5
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        ws = self.workspace(q.shape[1], q.shape[2], splits)
        capi.rbq_quant_attn_decode(self.desc, q, scale, causal, self.rot, out, splits, ws, mask)
        return out

    def append_attend(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
                      scale: Optional[float] = None, causal: bool = True, splits: int = 0,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """One decoding step: ``append(k, v)`` then ``attend(q)`` in one library
        call (the attention kernel writes the new rows itself where it can)."""
        n = k.shape[2]
        self.reserve(n)
        if scale is None:
            scale = self.desc.head_dim ** -0.5
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=self.device)
        after = capi.rbq_kv_cache.from_buffer_copy(self.desc)
        after.offset += n
        nb = capi.rbq_quant_attn_workspace_bytes(after, q.shape[1], q.shape[2], splits)
        ws = None
        if nb > 0:
            if self._ws is None or self._ws.numel() < nb:
                self._ws = torch.empty(nb, dtype=torch.uint8, device=self.device)
            ws = self._ws
        capi.rbq_kv_append_attn_decode(self.desc, k, v, q, scale, causal, self.rot, out, splits, ws)
        return out

    # -- batched verification of draft paths (mtp/kv_cache.py) -----------------
    def _regather(self, B: int, src_b0: int, src_b_step: int) -> None:
        """Replace the buffers by new ones of batch B, same capacity, whose
        batch entry b holds rows [0, offset) of entry src_b0 + b*src_b_step."""
        new = capi.rbq_kv_cache.from_buffer_copy(self.desc)
        new.B = B
        arrays = None
        if self.arrays is not None:
            arrays = self._alloc(self.capacity, B)
            self._bind(new, arrays, self.capacity)
            capi.rbq_kv_copy_batch(self.desc, src_b0, src_b_step, new)
        self.arrays, self.desc = arrays, new

    def tile(self, P: int) -> None:
        """``tile_caches`` for this cache: a batch-1 cache becomes batch P,
        every entry a copy of it (the page's state setter leaves buffers of
        exactly offset rows; here they keep the current capacity)."""
        if self.desc.B != 1:
            raise ValueError("tile needs a batch-1 cache")
        if P < 1:
            raise ValueError("P must be >= 1")
        self._regather(P, 0, 0)

    def commit_row(self, verified_len: int, accepted_len: int, row: int) -> None:
        """``commit_tree_row`` for this cache: trim the rejected suffix, then
        keep batch entry ``row`` (the winning path) as a batch-1 cache."""
        rejected = verified_len - accepted_len
        if rejected < 0:
            raise ValueError("accepted_len cannot exceed verified_len")
        if not 0 <= row < self.desc.B:
            raise ValueError(f"row {row} outside the batch of {self.desc.B}")
        if rejected:
            self.trim(rejected)
        self._regather(1, row, 0)

    # -- snapshots (the page's snapshot interface) ------------------------------
    @property
    def meta_state(self) -> tuple:
        """``meta_state``: group size and bit widths as strings."""
        d = self.desc
        return str(d.group_size), str(d.k_bits), str(d.v_bits)

    @property
    def state(self) -> Optional[dict]:
        """``state``: views of the six arrays' rows [0, offset) (None without
        buffers).  Views, not copies: :meth:`snapshot` makes the copy."""
        return None if self.arrays is None else self.rows()

    def snapshot(self) -> "CacheSnapshot":
        """Copy of the offset-prefix of the six buffers into buffers of their
        own (``_snapshot`` on the mtp/kv_cache.py page), by one device copy."""
        if self.arrays is None or self.offset == 0:
            return CacheSnapshot(None, None, self.meta_state)
        arrays = self._alloc(self.offset)
        desc = capi.rbq_kv_cache.from_buffer_copy(self.desc)
        desc.offset = 0
        self._bind(desc, arrays, self.offset)
        capi.rbq_kv_copy_prefix(self.desc, desc)
        return CacheSnapshot(arrays, desc, self.meta_state)

    def restore(self, snap: "CacheSnapshot") -> None:
        """``_restore``: the cache's rows [0, offset) and offset become the
        snapshot's; the snapshot is left as it is.  The copy goes into the
        cache's own buffers when they hold it (the page installs a fresh copy
        of exactly ``offset`` rows; rows and offset are the same either way,
        only the spare capacity differs), else into new buffers of exactly the
        snapshot's rows."""
        if snap.meta_state != self.meta_state:
            raise ValueError("snapshot of another cache configuration")
        if snap.desc is None:
            self.arrays = None
            self.desc.capacity = 0
            self.desc.offset = 0
            for name in capi_array_names():
                setattr(self.desc, name, None)
            return
        if self.arrays is None or self.capacity < snap.offset:
            new = self._alloc(snap.offset)
            desc = capi.rbq_kv_cache.from_buffer_copy(self.desc)
            self._bind(desc, new, snap.offset)
            capi.rbq_kv_copy_prefix(snap.desc, desc)
            self.arrays, self.desc = new, desc
        else:
            capi.rbq_kv_copy_prefix(snap.desc, self.desc)

    # -- inspection ------------------------------------------------------------
    def rows(self, upto: Optional[int] = None) -> dict:
        """Views of the six arrays' rows [0, upto or offset)."""
        n = self.offset if upto is None else upto
        return {k: a[:, :, :n] for k, a in self.arrays.items()}


def capi_array_names() -> tuple:
    """Names of the six buffer pointers in the cache descriptor."""
    return ("k_words", "k_scales", "k_biases", "v_words", "v_scales", "v_biases")


class CacheSnapshot:
    """A copy of a cache's offset-prefix: six device buffers of exactly
    ``offset`` rows with their descriptor, and the cache's meta state.
    ``desc`` is None for the empty marker (a cache without rows)."""

    def __init__(self, arrays: Optional[dict], desc, meta_state: tuple):
        self.arrays = arrays
        self.desc = desc
        self.meta_state = meta_state

    @property
    def offset(self) -> int:
        return 0 if self.desc is None else int(self.desc.offset)


def snapshot_caches(caches) -> list:
    """``_snapshot``: one snapshot per cache."""
    return [c.snapshot() for c in caches]


def restore_caches(caches, snaps) -> None:
    """``_restore``: each cache back to its snapshot."""
    for c, s in zip(caches, snaps):
        c.restore(s)


def commit_verified_snapshot(caches, snapshots, accepted_len: int,
                             verified_len: Optional[int] = None) -> bool:
    """``commit_verified_snapshot`` (page mtp/kv_cache.py): True without a
    restore when every verified token was accepted; False for accepted_len
    outside [1, len(snapshots)]; otherwise restore ``snapshots[accepted_len -
    1]`` (the snapshots taken after each verified token) and return True."""
    if verified_len is not None and accepted_len == verified_len:
        return True
    if accepted_len <= 0 or accepted_len > len(snapshots):
        return False
    restore_caches(caches, snapshots[accepted_len - 1])
    return True


def tile_caches(caches, P: int) -> None:
    """``tile_caches`` (page mtp/kv_cache.py): every batch-1 cache spread over
    P batch entries for a batched verification of P draft paths."""
    for c in caches:
        c.tile(P)


def commit_tree_row(caches, verified_len: int, accepted_len: int, row: int) -> bool:
    """``commit_tree_row`` for trimmable caches (page mtp/kv_cache.py): after a
    batched verification, trim the rejected suffix and keep path ``row`` as
    the batch-1 cache; ValueError when accepted_len > verified_len."""
    if verified_len - accepted_len < 0:
        raise ValueError("accepted_len cannot exceed verified_len")
    for c in caches:
        c.commit_row(verified_len, accepted_len, row)
    return True

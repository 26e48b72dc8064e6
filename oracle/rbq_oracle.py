"""Plain, slow, obviously correct CPU oracle (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP path.

Source of every definition: the page "mlx_streaming/core/cache/quant_kv.py"
(sparkle), sections "SO(4) block rotation" (``_quat_left``,
``_quat_right_conj``, ``build_block_so4``, ``rotate_last``), "asymmetric
quantized KV cache (K4/V3)" (``_packed_words``, ``AsymmetricQuantizedKVCache``:
``_init_quant``, ``update_and_fetch``, ``trim``) and "asymmetric quantized
SDPA" (``asym_quantized_sdpa``) and its snapshot interface (``state``,
``meta_state``); and the page "mlx_streaming/mtp/kv_cache.py",
``commit_verified_prefix``, ``_snapshot``, ``_restore``,
``commit_verified_snapshot``, ``tile_caches`` and ``commit_tree_row``.  The quantizer formula (scale = (max-min)/(2^bits-1),
bias = min, code = clip(round-half-even((x-bias)/scale))) and the little-endian
bit-stream packing are the ones the benchmark spec fixes; the pages call
``mx.quantize`` without defining it.

Readings taken where the pages leave a step open (each also listed in the
design notes):
  R1  the right-hand block matrix is used exactly as printed (it equals the
      transpose of the left-multiplication matrix);
  R2  quaternions are normalised and multiplied in fp64 and the block is
      rounded once to fp32 (the page does this in float32 through numpy);
  R3  rotations are fp64 sums of exact products in a fixed order, rounded
      once to fp32, and the rotated K/V are not rounded to the input dtype;
  R4  scale and bias are stored in the input dtype, and the codes are computed
      against the stored (rounded) scale and bias;
  R5  a zero scale divides by 1 (codes 0, dequant = bias);
  R6  attention accumulates in fp64 here (fp32 on the GPU) and returns fp32.

Variants beyond the default configuration (same pages): bit widths 2/3/4/5/6/8
(the width list in ``_packed_words``), any group size dividing head_dim (the
cache constructor's ``group_size``), head_dim 64/128/256, the two-sided block
rotation that the ``_quat_right_conj`` docstring describes (``mode=
"two_sided"``), and the page's own rotation precision (``round_rotated``: the
rotation entries and every rotated vector rounded to the input dtype, as
``rotate_last`` does with ``R.astype(x.dtype)``).
"""
from __future__ import annotations

import math

import numpy as np

GROUP = 64
STEP = 256  # cache growth step, AsymmetricQuantizedKVCache.step


# ---------------------------------------------------------------- rotation --

def quat_left(q) -> np.ndarray:
    """4x4 left-multiplication matrix of quaternion q = (w, x, y, z), entries as
    printed for ``_quat_left`` (page quant_kv.py, "SO(4) block rotation")."""
    w, x, y, z = (float(v) for v in q)
    return np.array([
        [w, -x, -y, -z],
        [x, w, -z, y],
        [y, z, w, -x],
        [z, -y, x, w],
    ], dtype=np.float64)


def quat_right_conj(q) -> np.ndarray:
    """4x4 matrix printed for ``_quat_right_conj`` (same page and section).

    Reading R1: the entries are taken as printed.  They equal
    ``quat_left(q).T``; the page's docstring describes a right
    multiplication by conj(q), which these entries do not implement."""
    w, x, y, z = (float(v) for v in q)
    return np.array([
        [w, x, y, z],
        [-x, w, z, -y],
        [-y, -z, w, x],
        [-z, y, -x, w],
    ], dtype=np.float64)


def quat_right_true_conj(q) -> np.ndarray:
    """4x4 matrix of v -> v (x) conj(q), the map the ``_quat_right_conj``
    docstring describes (quaternions as column vectors (w, x, y, z)).  Written
    out from the Hamilton product with p = conj(q) = (w, -x, -y, -z):
    v (x) p = (v0 p0 - v1 p1 - v2 p2 - v3 p3, v0 p1 + v1 p0 + v2 p3 - v3 p2,
               v0 p2 - v1 p3 + v2 p0 + v3 p1, v0 p3 + v1 p2 - v2 p1 + v3 p0)."""
    w, x, y, z = (float(v) for v in q)
    p0, p1, p2, p3 = w, -x, -y, -z
    return np.array([
        [p0, -p1, -p2, -p3],
        [p1, p0, p3, -p2],
        [p2, -p3, p0, p1],
        [p3, p2, -p1, p0],
    ], dtype=np.float64)


def normalize_quat(a) -> np.ndarray:
    """a / |a| in fp64: squares summed left to right, correctly rounded sqrt
    and division (reading R2)."""
    a0, a1, a2, a3 = (float(v) for v in a)
    n = math.sqrt(((a0 * a0 + a1 * a1) + a2 * a2) + a3 * a3)
    if n == 0.0:
        raise ValueError("zero-norm quaternion draw")
    return np.array([a0 / n, a1 / n, a2 / n, a3 / n], dtype=np.float64)


def matmul4_ordered(A: np.ndarray, Bm: np.ndarray) -> np.ndarray:
    """4x4 fp64 product with each entry summed over k = 0..3 in that order."""
    C = np.zeros((4, 4), dtype=np.float64)
    for i in range(4):
        for j in range(4):
            s = float(A[i, 0]) * float(Bm[0, j])
            for k in range(1, 4):
                s = s + float(A[i, k]) * float(Bm[k, j])
            C[i, j] = s
    return C


def rotation_blocks(draws: np.ndarray, mode: str = "printed") -> np.ndarray:
    """Blocks of the block-diagonal rotation (``build_block_so4``).

    draws: float32 ``[D/4, 2, 4]`` (left draw, right draw per block, in the
    page's draw order).  Returns float32 ``[D/4, 4, 4]``:
    block b = quat_left(qL) @ R(qR), qL/qR the normalised draws, computed in
    fp64 and rounded once to fp32 (reading R2), with R = the printed
    ``_quat_right_conj`` (mode "printed", reading R1) or the right
    multiplication by conj(qR) that its docstring describes (mode
    "two_sided")."""
    draws = np.asarray(draws, dtype=np.float32)
    if draws.ndim != 3 or draws.shape[1:] != (2, 4):
        raise ValueError("draws must be [D/4, 2, 4]")
    right = {"printed": quat_right_conj, "two_sided": quat_right_true_conj}[mode]
    out = np.empty((draws.shape[0], 4, 4), dtype=np.float32)
    for b in range(draws.shape[0]):
        qL = normalize_quat(draws[b, 0])
        qR = normalize_quat(draws[b, 1])
        out[b] = matmul4_ordered(quat_left(qL), right(qR)).astype(np.float32)
    return out


def dense_rotation(blocks: np.ndarray) -> np.ndarray:
    """The dense D x D block-diagonal matrix M (fp64) holding ``blocks`` on its
    diagonal, block b at rows/cols [4b, 4b+4) (``build_block_so4``)."""
    nb = blocks.shape[0]
    M = np.zeros((4 * nb, 4 * nb), dtype=np.float64)
    for b in range(nb):
        M[4 * b:4 * b + 4, 4 * b:4 * b + 4] = blocks[b]
    return M


def rotate(x: np.ndarray, blocks: np.ndarray) -> np.ndarray:
    """Row-vector rotation y = x @ M (``rotate_last``), reading R3:
    y[4b+j] = fp32(((x0*B[0,j] + x1*B[1,j]) + x2*B[2,j]) + x3*B[3,j]) in fp64,
    x_i = x[4b+i].  ``x`` holds fp16/bf16/fp32 values; returns float32."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    Bm = np.asarray(blocks, dtype=np.float64)
    xr = x.reshape(x.shape[:-1] + (D // 4, 4))
    y = xr[..., 0, None] * Bm[:, 0, :]
    y = y + xr[..., 1, None] * Bm[:, 1, :]
    y = y + xr[..., 2, None] * Bm[:, 2, :]
    y = y + xr[..., 3, None] * Bm[:, 3, :]
    return y.reshape(x.shape).astype(np.float32)


def inverse_rotate(y: np.ndarray, blocks: np.ndarray) -> np.ndarray:
    """z = y @ M^T (the inverse rotation of the attention output, page
    quant_kv.py design notes and ``asym_quantized_sdpa`` docstring):
    z[4b+i] = fp32(sum_{j=0..3} y[4b+j]*B[i,j]) in fp64, j in order."""
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    Bm = np.asarray(blocks, dtype=np.float64)
    yr = y.reshape(y.shape[:-1] + (D // 4, 4))
    z = yr[..., 0, None] * Bm[:, :, 0]
    z = z + yr[..., 1, None] * Bm[:, :, 1]
    z = z + yr[..., 2, None] * Bm[:, :, 2]
    z = z + yr[..., 3, None] * Bm[:, :, 3]
    return z.reshape(y.shape).astype(np.float32)


# --------------------------------------------------------------- quantizer --

def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to ``dtype`` ("bf16" or "f16"), round-half-even,
    and return them as float32 (exact).  bf16: keep the top 16 bits of the
    fp32 encoding after adding half an ulp (ties to even); f16: numpy's cast."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float32)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def quantize(y: np.ndarray, bits: int, dtype: str, group: int = GROUP):
    """Group-wise asymmetric affine quantizer (``mx.quantize`` as called in
    ``update_and_fetch``; formula fixed by the benchmark spec).

    y: float32 ``[..., D]``.  For each group of ``group`` consecutive values:
      mn, mx = min, max                                   (exact)
      s32    = fp32(fp32(mx - mn) / fp32(2^bits - 1))
      s, b   = s32 and mn rounded to ``dtype``            (reading R4)
      code   = clip(rint(fp32(fp32(y - b) / (s or 1))), 0, 2^bits - 1)   (R5)
    Returns (codes uint8 [..., D], scales float32 [..., D/group],
    biases float32 [..., D/group]); scales/biases hold ``dtype`` values."""
    y = np.asarray(y, dtype=np.float32)
    D = y.shape[-1]
    if D % group:
        raise ValueError("head_dim must be a multiple of the group size")
    g = y.reshape(y.shape[:-1] + (D // group, group))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    levels = np.float32(2 ** bits - 1)
    s32 = (mx - mn) / levels
    s = round_to_dtype(s32, dtype)
    b = round_to_dtype(mn, dtype)
    sdiv = np.where(s == np.float32(0), np.float32(1), s).astype(np.float32)
    q = (g - b[..., None]) / sdiv[..., None]
    codes = np.clip(np.rint(q), 0, 2 ** bits - 1).astype(np.uint8)
    return codes.reshape(y.shape), s, b


def dequantize(codes: np.ndarray, scales: np.ndarray, biases: np.ndarray,
               group: int = GROUP) -> np.ndarray:
    """x_hat = code * scale + bias of the code's group, in fp64."""
    c = np.asarray(codes, dtype=np.float64)
    D = c.shape[-1]
    cg = c.reshape(c.shape[:-1] + (D // group, group))
    x = cg * np.asarray(scales, np.float64)[..., None] + np.asarray(biases, np.float64)[..., None]
    return x.reshape(c.shape)


# ------------------------------------------------------------------ packing --

def packed_words(dim: int, bits: int) -> int:
    """uint32 words per packed row: dim*bits//32 (``_packed_words``)."""
    return dim * bits // 32


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Little-endian bit stream: bit t of code j sits at stream position
    p = bits*j + t, i.e. bit (p mod 32) of word p // 32."""
    c = np.asarray(codes, dtype=np.uint32)
    D = c.shape[-1]
    if (D * bits) % 32:
        raise ValueError("row does not fill whole words")
    stream = (c[..., :, None] >> np.arange(bits, dtype=np.uint32)) & np.uint32(1)
    stream = stream.reshape(c.shape[:-1] + (D * bits // 32, 32)).astype(np.uint64)
    words = (stream << np.arange(32, dtype=np.uint64)).sum(axis=-1)
    return words.astype(np.uint32)


def unpack(words: np.ndarray, bits: int, dim: int) -> np.ndarray:
    """Inverse of ``pack``."""
    w = np.asarray(words, dtype=np.uint32)
    stream = ((w[..., :, None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1))
    stream = stream.reshape(w.shape[:-1] + (w.shape[-1] * 32,))[..., :dim * bits]
    stream = stream.reshape(w.shape[:-1] + (dim, bits)).astype(np.uint32)
    codes = (stream << np.arange(bits, dtype=np.uint32)).sum(axis=-1)
    return codes.astype(np.uint8)


def rotate_for_cache(x: np.ndarray, blocks, dtype: str, round_rotated: bool = False) -> np.ndarray:
    """The rotation applied to q, k and v before they meet the cache.

    Default (reading R3): rotate(x, blocks), fp32.  With ``round_rotated``
    (the page's own precision in ``rotate_last``: ``x @ R.astype(x.dtype)``
    returns the input dtype), the result is rounded to ``dtype``; the caller
    passes blocks already rounded to ``dtype`` (``round_to_dtype(blocks)``).
    ``blocks`` None = identity (x unchanged)."""
    if blocks is None:
        return np.asarray(x, dtype=np.float32)
    y = rotate(x, blocks)
    return round_to_dtype(y, dtype) if round_rotated else y


def quantize_rows(x: np.ndarray, blocks, bits: int, dtype: str, group: int = GROUP,
                  round_rotated: bool = False):
    """Rotate (``blocks`` may be None = identity) then quantize and pack rows.
    Returns (words uint32, scales float32, biases float32)."""
    y = rotate_for_cache(x, blocks, dtype, round_rotated)
    codes, s, b = quantize(y, bits, dtype, group)
    return pack(codes, bits), s, b


# -------------------------------------------------------------------- cache --

def required_capacity(capacity: int, offset: int, n: int) -> int:
    """Capacity after ``update_and_fetch`` prepares room for n more rows
    (page quant_kv.py, ``AsymmetricQuantizedKVCache.update_and_fetch``, step 256):
    nothing changes while offset + n fits; otherwise ceil(n/256)*256 rows are
    added, after first cutting the buffer back to ``offset`` when ``offset``
    is not a multiple of 256.  ``capacity == 0`` means no buffer yet."""
    if n < 0 or offset < 0 or offset > capacity:
        raise ValueError("bad capacity/offset/n")
    if capacity > 0 and offset + n <= capacity:
        return capacity
    new_steps = (STEP + n - 1) // STEP * STEP
    if capacity == 0:
        return new_steps
    base = offset if offset % STEP != 0 else capacity
    return base + new_steps


class QuantKVCache:
    """Oracle of ``AsymmetricQuantizedKVCache`` (page quant_kv.py): six arrays
    (K words/scales/biases, V words/scales/biases) of shape [B, H, cap, .],
    ``offset`` rows valid.  Rows beyond ``offset`` are never read."""

    def __init__(self, k_bits: int = 4, v_bits: int = 3, dtype: str = "bf16",
                 group: int = GROUP, round_rotated: bool = False):
        self.k_bits, self.v_bits, self.dtype = k_bits, v_bits, dtype
        self.group, self.round_rotated = group, round_rotated
        self.offset = 0
        self.arrays = None  # dict name -> ndarray

    @property
    def capacity(self) -> int:
        return 0 if self.arrays is None else self.arrays["kw"].shape[2]

    def _grow(self, B, H, D, n):
        cap = required_capacity(self.capacity, self.offset, n)
        if cap == self.capacity:
            return
        shapes = {
            "kw": (packed_words(D, self.k_bits), np.uint32),
            "ks": (D // self.group, np.float32), "kb": (D // self.group, np.float32),
            "vw": (packed_words(D, self.v_bits), np.uint32),
            "vs": (D // self.group, np.float32), "vb": (D // self.group, np.float32),
        }
        new = {}
        for name, (w, dt) in shapes.items():
            a = np.zeros((B, H, cap, w), dtype=dt)
            if self.arrays is not None:
                keep = min(self.offset if self.offset % STEP else self.capacity, cap)
                a[:, :, :keep] = self.arrays[name][:, :, :keep]
            new[name] = a
        self.arrays = new

    def append(self, k: np.ndarray, v: np.ndarray, blocks) -> None:
        """``update_and_fetch``: rotate k/v (reading R3), quantize, write rows
        [offset, offset+n) and advance ``offset``."""
        B, H, n, D = k.shape
        self._grow(B, H, D, n)
        kw, ks, kb = quantize_rows(k, blocks, self.k_bits, self.dtype, self.group,
                                   self.round_rotated)
        vw, vs, vb = quantize_rows(v, blocks, self.v_bits, self.dtype, self.group,
                                   self.round_rotated)
        o = self.offset
        for name, val in (("kw", kw), ("ks", ks), ("kb", kb), ("vw", vw), ("vs", vs), ("vb", vb)):
            self.arrays[name][:, :, o:o + n] = val
        self.offset = o + n

    def trim(self, n: int) -> int:
        """``trim``: n' = min(offset, n); offset -= n'; returns n'."""
        if n < 0:
            raise ValueError("trim count must be >= 0")
        n = min(self.offset, n)
        self.offset -= n
        return n

    def dequant_kv(self, b: int, h: int):
        """Dequantised K and V rows [0, offset) of (b, h), fp64 [offset, D]."""
        a, o = self.arrays, self.offset
        D = a["ks"].shape[-1] * self.group
        kc = unpack(a["kw"][b, h, :o], self.k_bits, D)
        vc = unpack(a["vw"][b, h, :o], self.v_bits, D)
        return (dequantize(kc, a["ks"][b, h, :o], a["kb"][b, h, :o], self.group),
                dequantize(vc, a["vs"][b, h, :o], a["vb"][b, h, :o], self.group))


def cache_state(cache: QuantKVCache):
    """The snapshot interface's ``state`` getter (page quant_kv.py): the six
    arrays cut to ``offset`` rows.  Returned as copies: the page's slices are
    new arrays that the cache's later in-place writes cannot reach."""
    if cache.arrays is None:
        return None
    return {name: a[:, :, :cache.offset].copy() for name, a in cache.arrays.items()}


def set_cache_state(cache: QuantKVCache, state) -> None:
    """The ``state`` setter: the buffers become the given arrays and
    ``offset`` their row count (``None``: no buffers, offset 0)."""
    if state is None:
        cache.arrays, cache.offset = None, 0
        return
    cache.arrays = {name: a.copy() for name, a in state.items()}
    cache.offset = cache.arrays["kw"].shape[2]


def meta_state(cache: QuantKVCache):
    """``meta_state``: group size and bit widths as strings."""
    return str(cache.group), str(cache.k_bits), str(cache.v_bits)


def snapshot(caches):
    """``_snapshot`` (page mtp/kv_cache.py): per cache a copy of its state and
    its meta state; a cache without buffers gives the empty marker (None)."""
    return [(cache_state(c), meta_state(c)) for c in caches]


def restore(caches, snaps) -> None:
    """``_restore``: each cache receives a fresh copy of its snapshot's state
    (the snapshot itself stays untouched), or loses its buffers for the empty
    marker."""
    for c, (st, meta) in zip(caches, snaps):
        if meta != meta_state(c):
            raise ValueError("snapshot of another cache configuration")
        set_cache_state(c, st)


def commit_verified_snapshot(caches, snapshots, accepted_len: int,
                             verified_len=None) -> bool:
    """``commit_verified_snapshot``: nothing to do when every verified token
    was accepted; False for accepted_len outside [1, len(snapshots)];
    otherwise restore the snapshot taken after accepted_len tokens."""
    if verified_len is not None and accepted_len == verified_len:
        return True
    if accepted_len <= 0 or accepted_len > len(snapshots):
        return False
    restore(caches, snapshots[accepted_len - 1])
    return True


def commit_verified_prefix(cache: QuantKVCache, verified_len: int, accepted_len: int) -> int:
    """Trimmable branch of ``commit_verified_prefix`` (page mtp/kv_cache.py):
    ValueError when accepted_len > verified_len, else trim the rejected suffix."""
    rejected = verified_len - accepted_len
    if rejected < 0:
        raise ValueError("accepted_len cannot exceed verified_len")
    return cache.trim(rejected) if rejected else 0


# ---------------------------------------------------------------- attention --

def attention_row(q_row: np.ndarray, khat: np.ndarray, vhat: np.ndarray, n_keys: int,
                  scale: float, blocks, mask_row=None, dtype: str = "bf16",
                  round_rotated: bool = False) -> np.ndarray:
    """One query row of ``asym_quantized_sdpa`` followed by the inverse rotation.

    q_row: [D] input-dtype values (unrotated); khat/vhat: fp64 dequantised
    rows; keys [0, n_keys) are visible.  q' = rotate(q) (fp32), then in fp64:
    scores = (q' * scale) . khat_t, max-subtracted softmax, o = sum p_t vhat_t;
    returns inverse_rotate(fp32(o)) (or fp32(o) when blocks is None).

    mask_row (the SDPA's array mask, one row over keys [0, n_keys)): boolean,
    a false entry's score becomes the most negative finite value (the page's
    ``finfo.min`` fill: such a key gets weight 0 unless every key of the row is
    masked, when the softmax of equal scores weights all keys alike); or
    floating point, added to the scaled scores.  ``round_rotated``: q' is
    rounded to ``dtype`` (``rotate_for_cache``); the output stays fp32."""
    qr = rotate_for_cache(q_row, blocks, dtype, round_rotated)
    qs = qr.astype(np.float64) * float(scale)
    sc = khat[:n_keys] @ qs
    if mask_row is not None:
        mrow = np.asarray(mask_row)[:n_keys]
        if mrow.dtype == np.bool_:
            sc = np.where(mrow, sc, np.finfo(np.float64).min)
        else:
            sc = sc + mrow.astype(np.float64)
    m = sc.max()
    p = np.exp(sc - m)
    o = (p @ vhat[:n_keys]) / p.sum()
    o32 = o.astype(np.float32)
    return o32 if blocks is None else inverse_rotate(o32, blocks)


def attention(q: np.ndarray, cache: QuantKVCache, scale: float, causal: bool, blocks,
              rows=None, mask=None) -> np.ndarray:
    """Fused decode/verify attention over the cache (``asym_quantized_sdpa``):
    q: [B, Hq, L, D]; q head h reads kv head h // (Hq/Hkv); with ``causal``,
    row i of the L-block sees keys t <= offset - L + i; ``mask`` (optional,
    broadcastable to [B, Hq, L, offset], boolean or additive) applies to the
    keys as well.  Returns float32 [B, Hq, L, D] (only ``rows`` = iterable of
    (b, h, i) are filled if given, the rest stay NaN)."""
    B, Hq, L, D = q.shape
    Hkv = cache.arrays["kw"].shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    n_rep = Hq // Hkv
    T = cache.offset
    if L < 1 or L > T:
        raise ValueError("need 1 <= L <= offset")
    if mask is not None:
        mask = np.broadcast_to(np.asarray(mask), (B, Hq, L, np.asarray(mask).shape[-1]))
        if mask.shape[-1] < T:
            raise ValueError("the mask must cover keys [0, offset)")
    out = np.full((B, Hq, L, D), np.nan, dtype=np.float32)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(L)]
    deq = {}
    for (b, h, i) in rows:
        kvh = h // n_rep
        if (b, kvh) not in deq:
            deq = {(b, kvh): cache.dequant_kv(b, kvh)}
        khat, vhat = deq[(b, kvh)]
        n_keys = T - L + i + 1 if causal else T
        mrow = None if mask is None else mask[b, h, i]
        out[b, h, i] = attention_row(q[b, h, i], khat, vhat, n_keys, scale, blocks, mrow,
                                     cache.dtype, cache.round_rotated)
    return out


def tile_cache(cache: QuantKVCache, P: int) -> None:
    """``tile_caches`` (page mtp/kv_cache.py) for one cache: its batch-1 state
    repeated P times along the batch axis, through the state setter (so the
    buffers hold exactly ``offset`` rows)."""
    st = cache_state(cache)
    if st is None:
        return
    if st["kw"].shape[0] != 1:
        raise ValueError("tile_caches needs batch-1 caches")
    set_cache_state(cache, {name: np.repeat(a, P, axis=0) for name, a in st.items()})


def commit_tree_row(caches, verified_len: int, accepted_len: int, row: int) -> bool:
    """``commit_tree_row`` for trimmable caches (page mtp/kv_cache.py): trim the
    rejected suffix, then keep batch row ``row`` (the winning path) as a
    batch-1 cache."""
    rejected = verified_len - accepted_len
    if rejected < 0:
        raise ValueError("accepted_len cannot exceed verified_len")
    for c in caches:
        if rejected:
            c.trim(rejected)
        st = cache_state(c)
        if st is not None:
            set_cache_state(c, {name: a[row:row + 1] for name, a in st.items()})
    return True

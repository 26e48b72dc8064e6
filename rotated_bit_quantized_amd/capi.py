"""ctypes binding of librbq (the C ABI in include/rbq.h): argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of the method: it checks Python-side types, passes device
pointers, sizes and torch's current HIP stream, and turns a negative status
into :class:`RbqError`.  All device work runs in the library's HIP kernels.

The library is loaded from the package directory (``librbq.so``, built in-tree
by ``rotated_bit_quantized_amd/csrc/build.py``).  There is no fallback: if it
is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p, POINTER

import numpy as np
import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librbq.so")

RBQ_OK = 0
RBQ_EINVAL = -1
RBQ_EUNSUPPORTED = -2
RBQ_ECAPACITY = -3
RBQ_ERANGE = -4
RBQ_EWORKSPACE = -5
RBQ_EHIP = -6
RBQ_ESCRATCH = -7

RBQ_SCRATCH_BYTES = 8 << 20  # fixed scratch array of rbq_quant_attn_decode_noalloc, per device

RBQ_F16 = 1
RBQ_BF16 = 2

RBQ_FLAG_ROUND_ROTATED = 1

RBQ_ROT_PRINTED = 0
RBQ_ROT_TWO_SIDED = 1

RBQ_MASK_NONE = 0
RBQ_MASK_BOOL = 1
RBQ_MASK_ADD_F32 = 2
RBQ_MASK_ADD_DTYPE = 3

DTYPE_CODES = {torch.float16: RBQ_F16, torch.bfloat16: RBQ_BF16}


class RbqError(RuntimeError):
    """A negative status returned by librbq."""

    def __init__(self, func: str, status: int):
        self.status = status
        msg = _lib.rbq_status_string(status).decode()
        if status == RBQ_EHIP:
            msg += f" (hipError_t {_lib.rbq_last_hip_error()})"
        super().__init__(f"{func}: {msg} [{status}]")


class rbq_kv_cache(ctypes.Structure):
    """Mirror of the C descriptor ``rbq_kv_cache``."""

    _fields_ = [
        ("B", c_int32), ("H_kv", c_int32), ("head_dim", c_int32), ("group_size", c_int32),
        ("k_bits", c_int32), ("v_bits", c_int32), ("dtype", c_int32), ("flags", c_int32),
        ("capacity", c_int64), ("offset", c_int64),
        ("k_words", c_void_p), ("k_scales", c_void_p), ("k_biases", c_void_p),
        ("v_words", c_void_p), ("v_scales", c_void_p), ("v_biases", c_void_p),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python rotated_bit_quantized_amd/csrc/build.py` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER(rbq_kv_cache)
    sigs = {
        "rbq_rotation_build": (c_int32, [c_void_p, c_int32, c_void_p]),
        "rbq_rotation_build_mode": (c_int32, [c_void_p, c_int32, c_int32, c_void_p]),
        "rbq_rotation_round": (c_int32, [c_void_p, c_int32, c_int32]),
        "rbq_kv_required_capacity": (c_int64, [c_int64, c_int64, c_int64]),
        "rbq_kv_grow": (c_int32, [P, P, c_void_p]),
        "rbq_kv_copy_prefix": (c_int32, [P, P, c_void_p]),
        "rbq_kv_copy_batch": (c_int32, [P, c_int32, c_int32, P, c_void_p]),
        "rbq_kv_quant_append": (c_int32, [P, c_void_p, c_void_p, c_int64, c_void_p, c_void_p]),
        "rbq_kv_trim": (c_int64, [P, c_int64]),
        "rbq_kv_commit_verified": (c_int64, [P, c_int64, c_int64]),
        "rbq_quant_attn_splits": (c_int32, [P, c_int32, c_int32]),
        "rbq_quant_attn_workspace_bytes": (c_size_t, [P, c_int32, c_int32, c_int32]),
        "rbq_quant_attn_decode": (c_int32, [P, c_void_p, c_int32, c_int32, c_float, c_int32,
                                            c_void_p, c_void_p, c_int32, c_void_p, c_size_t,
                                            c_void_p]),
        "rbq_quant_attn_decode_noalloc": (c_int32, [P, c_void_p, c_int32, c_int32, c_float,
                                                    c_int32, c_void_p, c_void_p, c_int32,
                                                    c_void_p]),
        "rbq_kv_append_attn_decode": (c_int32, [P, c_void_p, c_void_p, c_int64, c_void_p, c_int32,
                                                c_int32, c_float, c_int32, c_void_p, c_void_p,
                                                c_int32, c_void_p, c_size_t, c_void_p]),
        "rbq_quant_attn_decode_mask": (c_int32, [P, c_void_p, c_int32, c_int32, c_float, c_int32,
                                                 c_void_p, c_int32, c_int64, c_int64, c_int64,
                                                 c_void_p, c_void_p, c_int32, c_void_p, c_size_t,
                                                 c_void_p]),
        "rbq_status_string": (ctypes.c_char_p, [c_int32]),
        "rbq_last_hip_error": (c_int32, []),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    """The loaded librbq handle."""
    return _lib


def _check(func: str, status: int) -> int:
    if status < 0:
        raise RbqError(func, int(status))
    return int(status)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev_ptr(t: torch.Tensor, dtype=None, name: str = "tensor") -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


# ---------------------------------------------------------------- host calls --

def rbq_rotation_build(draws: np.ndarray) -> np.ndarray:
    """Blocks ``float32 [D/4, 4, 4]`` of the SO(4) block rotation from the raw
    quaternion draws ``float32 [D/4, 2, 4]`` (host only)."""
    d = np.ascontiguousarray(draws, dtype=np.float32)
    if d.ndim != 3 or d.shape[1:] != (2, 4):
        raise ValueError("draws must be float32 [D/4, 2, 4]")
    out = np.empty((d.shape[0], 4, 4), dtype=np.float32)
    _check("rbq_rotation_build",
           _lib.rbq_rotation_build(d.ctypes.data, 4 * d.shape[0], out.ctypes.data))
    return out


def rbq_rotation_build_mode(draws: np.ndarray, mode: int) -> np.ndarray:
    """As :func:`rbq_rotation_build` with the right factor chosen by ``mode``
    (RBQ_ROT_PRINTED or RBQ_ROT_TWO_SIDED)."""
    d = np.ascontiguousarray(draws, dtype=np.float32)
    if d.ndim != 3 or d.shape[1:] != (2, 4):
        raise ValueError("draws must be float32 [D/4, 2, 4]")
    out = np.empty((d.shape[0], 4, 4), dtype=np.float32)
    _check("rbq_rotation_build_mode",
           _lib.rbq_rotation_build_mode(d.ctypes.data, 4 * d.shape[0], int(mode), out.ctypes.data))
    return out


def rbq_rotation_round(blocks: np.ndarray, dtype: int) -> np.ndarray:
    """A copy of the blocks ``float32 [D/4, 4, 4]`` with every entry rounded
    half to even to the cache dtype (RBQ_F16 or RBQ_BF16), host only."""
    b = np.array(blocks, dtype=np.float32, order="C", copy=True)
    if b.ndim != 3 or b.shape[1:] != (4, 4):
        raise ValueError("blocks must be float32 [D/4, 4, 4]")
    _check("rbq_rotation_round", _lib.rbq_rotation_round(b.ctypes.data, 4 * b.shape[0], int(dtype)))
    return b


def rbq_kv_required_capacity(capacity: int, offset: int, n: int) -> int:
    return _check("rbq_kv_required_capacity", _lib.rbq_kv_required_capacity(capacity, offset, n))


def rbq_kv_trim(desc: rbq_kv_cache, n: int) -> int:
    return _check("rbq_kv_trim", _lib.rbq_kv_trim(ctypes.byref(desc), n))


def rbq_kv_commit_verified(desc: rbq_kv_cache, verified_len: int, accepted_len: int) -> int:
    return _check("rbq_kv_commit_verified",
                  _lib.rbq_kv_commit_verified(ctypes.byref(desc), verified_len, accepted_len))


# -------------------------------------------------------------- device calls --

def rbq_kv_grow(src: rbq_kv_cache, dst: rbq_kv_cache) -> None:
    _check("rbq_kv_grow", _lib.rbq_kv_grow(ctypes.byref(src), ctypes.byref(dst), _stream()))


def rbq_kv_copy_prefix(src: rbq_kv_cache, dst: rbq_kv_cache) -> None:
    """Rows [0, src.offset) of the six arrays into dst; dst.offset = src.offset."""
    _check("rbq_kv_copy_prefix",
           _lib.rbq_kv_copy_prefix(ctypes.byref(src), ctypes.byref(dst), _stream()))


def rbq_kv_copy_batch(src: rbq_kv_cache, src_b0: int, src_b_step: int, dst: rbq_kv_cache) -> None:
    """Destination batch entry b <- rows [0, src.offset) of source entry
    src_b0 + b * src_b_step; dst.offset = src.offset."""
    _check("rbq_kv_copy_batch", _lib.rbq_kv_copy_batch(ctypes.byref(src), int(src_b0),
                                                       int(src_b_step), ctypes.byref(dst),
                                                       _stream()))


def rbq_kv_quant_append(desc: rbq_kv_cache, k: torch.Tensor, v: torch.Tensor,
                        rot_blocks) -> None:
    """k, v: device ``[B, H_kv, n, head_dim]`` in the cache dtype; rot_blocks:
    device float32 ``[D/4, 4, 4]`` or None.  Advances ``desc.offset`` by n."""
    if k.shape != v.shape or k.dim() != 4:
        raise ValueError("k and v must both be [B, H_kv, n, head_dim]")
    if (k.shape[0], k.shape[1], k.shape[3]) != (desc.B, desc.H_kv, desc.head_dim):
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match the cache")
    dt = _TORCH_OF[desc.dtype]
    kp = _dev_ptr(k, dt, "k")
    vp = _dev_ptr(v, dt, "v")
    rp = None if rot_blocks is None else _dev_ptr(rot_blocks, torch.float32, "rot_blocks")
    _check("rbq_kv_quant_append",
           _lib.rbq_kv_quant_append(ctypes.byref(desc), kp, vp, k.shape[2], rp, _stream()))


def rbq_quant_attn_splits(desc: rbq_kv_cache, H_q: int, L: int) -> int:
    return _check("rbq_quant_attn_splits", _lib.rbq_quant_attn_splits(ctypes.byref(desc), H_q, L))


def rbq_quant_attn_workspace_bytes(desc: rbq_kv_cache, H_q: int, L: int, splits: int = 0) -> int:
    return int(_lib.rbq_quant_attn_workspace_bytes(ctypes.byref(desc), H_q, L, splits))


def _mask_args(desc: rbq_kv_cache, mask, B: int, H_q: int, L: int):
    """(pointer, type, stride_b, stride_h, stride_l) of an optional mask
    tensor broadcastable to [B, H_q, L, keys]: bool/uint8 (nonzero = keep),
    float32 or the cache dtype (added to the scaled scores)."""
    if mask is None:
        return None, RBQ_MASK_NONE, 0, 0, 0
    if not mask.is_cuda:
        raise ValueError("mask must be a device (HIP) tensor")
    if mask.dim() == 2:
        mask = mask[None, None]
    if mask.dim() != 4:
        raise ValueError("mask must be [L, keys] or [B|1, H_q|1, L, keys]")
    m = mask.expand(B, H_q, L, mask.shape[-1])
    if m.shape[-1] < desc.offset:
        raise ValueError(f"mask covers {m.shape[-1]} keys, the cache holds {desc.offset}")
    if m.stride(-1) != 1:
        raise ValueError("the mask's key axis must be contiguous")
    if mask.dtype in (torch.bool, torch.uint8):
        mt = RBQ_MASK_BOOL
    elif mask.dtype == torch.float32:
        mt = RBQ_MASK_ADD_F32
    elif mask.dtype == _TORCH_OF[desc.dtype]:
        mt = RBQ_MASK_ADD_DTYPE
    else:
        raise ValueError(f"mask dtype {mask.dtype} is not supported")
    return m.data_ptr(), mt, m.stride(0), m.stride(1), m.stride(2)


def rbq_quant_attn_decode(desc: rbq_kv_cache, q: torch.Tensor, scale: float, causal: bool,
                          rot_blocks, out: torch.Tensor, splits: int = 0,
                          ws: torch.Tensor = None, mask: torch.Tensor = None) -> None:
    """q: device ``[B, H_q, L, head_dim]`` in the cache dtype; out: device
    float32 of the same shape (written); ws: device workspace of at least
    ``rbq_quant_attn_workspace_bytes`` bytes (None when that is 0); mask:
    optional device tensor broadcastable to ``[B, H_q, L, keys]`` (keys >=
    offset): bool/uint8 keeps where nonzero, float32 or the cache dtype is
    added to the scaled scores (calls rbq_quant_attn_decode_mask)."""
    if q.dim() != 4 or q.shape[0] != desc.B or q.shape[3] != desc.head_dim:
        raise ValueError(f"q shape {tuple(q.shape)} does not match the cache")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    qp = _dev_ptr(q, _TORCH_OF[desc.dtype], "q")
    op = _dev_ptr(out, torch.float32, "out")
    rp = None if rot_blocks is None else _dev_ptr(rot_blocks, torch.float32, "rot_blocks")
    wp, wn = None, 0
    if ws is not None:
        wp, wn = _dev_ptr(ws, None, "ws"), ws.numel() * ws.element_size()
    if mask is None:
        _check("rbq_quant_attn_decode",
               _lib.rbq_quant_attn_decode(ctypes.byref(desc), qp, q.shape[1], q.shape[2],
                                          float(scale), 1 if causal else 0, rp, op, int(splits),
                                          wp, wn, _stream()))
        return
    mp, mt, sb, sh, sl = _mask_args(desc, mask, q.shape[0], q.shape[1], q.shape[2])
    _check("rbq_quant_attn_decode_mask",
           _lib.rbq_quant_attn_decode_mask(ctypes.byref(desc), qp, q.shape[1], q.shape[2],
                                           float(scale), 1 if causal else 0, mp, mt, sb, sh, sl,
                                           rp, op, int(splits), wp, wn, _stream()))


def rbq_quant_attn_decode_noalloc(desc: rbq_kv_cache, q: torch.Tensor, scale: float,
                                  causal: bool, rot_blocks, out: torch.Tensor,
                                  splits: int = 0) -> None:
    """rbq_quant_attn_decode with the split records in the library's fixed
    device scratch array (no workspace argument; the call allocates nothing).
    Calls that overlap on one device share that array and must not overlap."""
    if q.dim() != 4 or q.shape[0] != desc.B or q.shape[3] != desc.head_dim:
        raise ValueError(f"q shape {tuple(q.shape)} does not match the cache")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    qp = _dev_ptr(q, _TORCH_OF[desc.dtype], "q")
    op = _dev_ptr(out, torch.float32, "out")
    rp = None if rot_blocks is None else _dev_ptr(rot_blocks, torch.float32, "rot_blocks")
    _check("rbq_quant_attn_decode_noalloc",
           _lib.rbq_quant_attn_decode_noalloc(ctypes.byref(desc), qp, q.shape[1], q.shape[2],
                                              float(scale), 1 if causal else 0, rp, op,
                                              int(splits), _stream()))


def rbq_kv_append_attn_decode(desc: rbq_kv_cache, k: torch.Tensor, v: torch.Tensor,
                              q: torch.Tensor, scale: float, causal: bool, rot_blocks,
                              out: torch.Tensor, splits: int = 0,
                              ws: torch.Tensor = None) -> None:
    """rbq_kv_quant_append(desc, k, v) then rbq_quant_attn_decode(desc, q, ...)
    as one call (one launch fewer where the attention kernel writes the rows
    itself).  ws: at least ``rbq_quant_attn_workspace_bytes`` of the cache
    after the append.  Advances ``desc.offset`` by n."""
    if k.shape != v.shape or k.dim() != 4:
        raise ValueError("k and v must both be [B, H_kv, n, head_dim]")
    if (k.shape[0], k.shape[1], k.shape[3]) != (desc.B, desc.H_kv, desc.head_dim):
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match the cache")
    if q.dim() != 4 or q.shape[0] != desc.B or q.shape[3] != desc.head_dim:
        raise ValueError(f"q shape {tuple(q.shape)} does not match the cache")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    dt = _TORCH_OF[desc.dtype]
    kp = _dev_ptr(k, dt, "k")
    vp = _dev_ptr(v, dt, "v")
    qp = _dev_ptr(q, dt, "q")
    op = _dev_ptr(out, torch.float32, "out")
    rp = None if rot_blocks is None else _dev_ptr(rot_blocks, torch.float32, "rot_blocks")
    wp, wn = None, 0
    if ws is not None:
        wp, wn = _dev_ptr(ws, None, "ws"), ws.numel() * ws.element_size()
    _check("rbq_kv_append_attn_decode",
           _lib.rbq_kv_append_attn_decode(ctypes.byref(desc), kp, vp, k.shape[2], qp, q.shape[1],
                                          q.shape[2], float(scale), 1 if causal else 0, rp, op,
                                          int(splits), wp, wn, _stream()))


def prepare_append_attn_decode(desc: rbq_kv_cache, k: torch.Tensor, v: torch.Tensor,
                               q: torch.Tensor, scale: float, causal: bool, rot_blocks,
                               out: torch.Tensor, splits: int = 0, ws: torch.Tensor = None):
    """``rbq_kv_append_attn_decode`` with its arguments checked and marshalled
    once, for a loop that repeats the same step on caches of ``desc``'s shape
    (the tensors must stay alive and in place; the stream is the current one
    now).  Returns ``call(desc)``, which makes the library call on that cache
    descriptor and raises on a nonzero status."""
    if k.shape != v.shape or k.dim() != 4:
        raise ValueError("k and v must both be [B, H_kv, n, head_dim]")
    if (k.shape[0], k.shape[1], k.shape[3]) != (desc.B, desc.H_kv, desc.head_dim):
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match the cache")
    if q.dim() != 4 or q.shape[0] != desc.B or q.shape[3] != desc.head_dim:
        raise ValueError(f"q shape {tuple(q.shape)} does not match the cache")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    dt = _TORCH_OF[desc.dtype]
    args = (_dev_ptr(k, dt, "k"), _dev_ptr(v, dt, "v"), k.shape[2], _dev_ptr(q, dt, "q"),
            q.shape[1], q.shape[2], float(scale), 1 if causal else 0,
            None if rot_blocks is None else _dev_ptr(rot_blocks, torch.float32, "rot_blocks"),
            _dev_ptr(out, torch.float32, "out"), int(splits),
            None if ws is None else _dev_ptr(ws, None, "ws"),
            0 if ws is None else ws.numel() * ws.element_size(), _stream())
    fn = _lib.rbq_kv_append_attn_decode

    def call(d: rbq_kv_cache) -> None:
        st = fn(ctypes.byref(d), *args)
        if st != RBQ_OK:
            _check("rbq_kv_append_attn_decode", st)

    return call


_TORCH_OF = {RBQ_F16: torch.float16, RBQ_BF16: torch.bfloat16}

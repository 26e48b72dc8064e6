"""Pure-Python loop twin of the oracle, for tiny inputs (TEST INFRASTRUCTURE ONLY).

It restates the same definitions as ``rbq_oracle`` with scalar loops, Python
floats and explicit fp32 rounding of every fp32 operation (an fp64 result of
one +, -, * or / of fp32 operands, rounded once to fp32, is the correctly
rounded fp32 result).  No numpy reductions are used, so a vectorisation or
axis mistake in ``rbq_oracle`` shows up as a disagreement.  Only ``tests/``
use it.
"""
from __future__ import annotations

import math
import struct


def f32(x: float) -> float:
    """Round a Python float (fp64) to the nearest fp32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bf16(x: float) -> float:
    """Round an fp32 value to bf16 (ties to even) by its bit pattern."""
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", u))[0]


def f16(x: float) -> float:
    """Round an fp32 value to IEEE half (ties to even) via struct's 'e' format."""
    return struct.unpack("<e", struct.pack("<e", x))[0]


def hamilton(p, q):
    """Hamilton product p*q of quaternions (w, x, y, z), from i^2=j^2=k^2=ijk=-1."""
    pw, px, py, pz = p
    qw, qx, qy, qz = q
    return (pw * qw - px * qx - py * qy - pz * qz,
            pw * qx + px * qw + py * qz - pz * qy,
            pw * qy - px * qz + py * qw + pz * qx,
            pw * qz + px * qy - py * qx + pz * qw)


def rotate_row(x, blocks):
    """y = x @ M for one row, fp64 sum of exact products per 4-block, in order."""
    y = []
    for b in range(len(x) // 4):
        for j in range(4):
            s = 0.0
            for i in range(4):
                s += float(x[4 * b + i]) * float(blocks[b][i][j])
            y.append(f32(s))
    return y


def inverse_rotate_row(y, blocks):
    z = []
    for b in range(len(y) // 4):
        for i in range(4):
            s = 0.0
            for j in range(4):
                s += float(y[4 * b + j]) * float(blocks[b][i][j])
            z.append(f32(s))
    return z


def quantize_row(y, bits: int, dtype: str, group: int = 64):
    """Scalar-loop quantizer of one row (same definition as rbq_oracle.quantize)."""
    rnd = bf16 if dtype == "bf16" else f16
    levels = float(2 ** bits - 1)
    codes, scales, biases = [], [], []
    for g0 in range(0, len(y), group):
        grp = [f32(v) for v in y[g0:g0 + group]]
        mn = grp[0]
        mx = grp[0]
        for v in grp[1:]:
            if v < mn:
                mn = v
            if v > mx:
                mx = v
        s32 = f32(f32(mx - mn) / levels)
        s = rnd(s32)
        b = rnd(mn)
        sdiv = s if s != 0.0 else 1.0
        for v in grp:
            t = f32(f32(v - b) / sdiv)
            c = round(t)  # Python's round(): ties to even
            c = max(0, min(int(c), 2 ** bits - 1))
            codes.append(c)
        scales.append(s)
        biases.append(b)
    return codes, scales, biases


def pack_row(codes, bits: int):
    """Character-level bit string packer: write every code's bits LSB first,
    cut the string into 32-character words, read each word LSB first."""
    stream = "".join(format(c, "0{}b".format(bits))[::-1] for c in codes)
    words = []
    for w0 in range(0, len(stream), 32):
        words.append(int(stream[w0:w0 + 32][::-1], 2))
    return words


def unpack_row(words, bits: int, dim: int):
    stream = "".join(format(w, "032b")[::-1] for w in words)
    return [int(stream[bits * j:bits * j + bits][::-1], 2) for j in range(dim)]


def attention_row(q, keys, vals, n_keys: int, scale: float, blocks):
    """One query row over dequantised fp64 rows, pure loops and math.exp."""
    qr = [float(v) for v in q] if blocks is None else rotate_row(q, blocks)
    qs = [v * scale for v in qr]
    scores = []
    for t in range(n_keys):
        s = 0.0
        for d in range(len(qs)):
            s += qs[d] * keys[t][d]
        scores.append(s)
    m = max(scores)
    ps = [math.exp(s - m) for s in scores]
    tot = sum(ps)
    o = []
    for d in range(len(qs)):
        acc = 0.0
        for t in range(n_keys):
            acc += ps[t] * vals[t][d]
        o.append(f32(acc / tot))
    return o if blocks is None else inverse_rotate_row(o, blocks)


def dequant_row(codes, scales, biases, group: int = 64):
    return [codes[d] * scales[d // group] + biases[d // group] for d in range(len(codes))]

"""Hand-built bf16 tensors that sit on the format's decision points.

Pure input construction: values are placed at E2M1 / E4M3 midpoints, their
bf16 neighbours, subnormal and zero block scales, saturation and signed
zeros.  No quantization arithmetic happens here; each case carries the static
global scale it is meant to be quantized under (None = dynamic).
"""
from __future__ import annotations

import numpy as np

from workloads import to_bf16_bits

_E2M1_MIDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def _bf16_neighbours(v):
    b = int(to_bf16_bits(np.array([v], np.float32))[0])
    return [b - 1, b, b + 1]


def e2m1_ties():
    """Static Sg = 1 and a 6 in every block: t = 6, s = 1, d = 1, so every
    element's ratio is the element itself.  Blocks hold each E2M1 midpoint and
    its bf16 neighbours, both signs."""
    six = int(to_bf16_bits(np.array([6.0], np.float32))[0])
    vals = []
    for m in _E2M1_MIDS + [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]:
        vals.extend(b for b in _bf16_neighbours(m) if b <= six)   # keep every block max at 6
    vals = np.array(vals, np.uint16)
    vals = np.concatenate([vals, vals | 0x8000])
    blocks = []
    for i in range(0, len(vals), 15):
        chunk = list(vals[i:i + 15])
        chunk += [0] * (15 - len(chunk))
        blocks.append([six] + chunk)
    return np.array(blocks, np.uint16).reshape(1, -1), 1.0


def e4m3_ties():
    """Static Sg = fl(1/6): t = fl(6 * Sg) = 1, so the block scale ratio is the
    block maximum itself.  Block maxima sit on E4M3 midpoints (and bf16
    neighbours) such as 1.0625 and 1.1875; the rest of the block is small."""
    sg = float(np.float32(1.0) / np.float32(6.0))
    maxima = []
    for m in [1.0625, 1.1875, 2.125, 0.53125, 3.0 * 2.0 ** -10, 2.0 ** -10, 7.5 * 2.0 ** -9, 17.0, 240.0,
              448.0, 464.0, 500.0]:
        maxima.extend(_bf16_neighbours(m))
    rows = []
    for mb in maxima:
        blk = [mb] + [int(to_bf16_bits(np.array([0.001 * (k + 1)], np.float32))[0]) for k in range(15)]
        rows.extend(blk)
    return np.array(rows, np.uint16).reshape(1, -1), sg


def scale_edge_cases():
    """Dynamic mode: one block carries the tensor amax (scale 448); others are
    tiny so their scales are subnormal E4M3 or zero; one block is all zero,
    one all negative zero, one a single nonzero element."""
    rng = np.random.default_rng(123)
    rows = []
    big = rng.standard_normal(16).astype(np.float32)
    big[3] = 40.0
    rows.append(big)
    for f in [2.0 ** -6, 2.0 ** -8, 2.0 ** -9, 3.0 * 2.0 ** -10, 2.0 ** -11, 2.0 ** -14]:
        # block maximum = 40 * f / 448 * 6 ... a spread of small block maxima
        blk = rng.standard_normal(16).astype(np.float32) * np.float32(40.0 * f)
        rows.append(blk)
    rows.append(np.zeros(16, np.float32))
    rows.append(-np.zeros(16, np.float32))
    single = np.zeros(16, np.float32)
    single[7] = -0.37
    rows.append(single)
    # bf16 extremes inside one block next to the amax block
    tiny = np.zeros(16, np.float32)
    tiny[0] = 2.0 ** -133       # smallest bf16 subnormal
    tiny[1] = -(2.0 ** -126)
    rows.append(tiny)
    return to_bf16_bits(np.concatenate(rows)).reshape(1, -1), None


def saturation(static_scale: float = 1e-3):
    """Static scale far too small: block scales saturate at 448 and codes at 6."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 64)).astype(np.float32) * np.float32(10.0)
    return to_bf16_bits(x), static_scale


def _tie_block(d, bmax, rng):
    """A block holding bmax and the E2M1 midpoints of divisor d (both signs,
    with bf16 neighbours where d is not a power of two)."""
    vals = [bmax]
    for m in _E2M1_MIDS:
        vals.append(m * d)
        vals.append(-m * d)
    while len(vals) < 16:
        vals.append(float(rng.uniform(-1.0, 1.0)) * bmax)
    return np.array(vals[:16], np.float64)


def extreme_global_scales():
    """Static global scales that put block divisors d = s * Sg at the edges of
    the range where a quantizer may divide through a reciprocal, on both sides
    of it: Sg = 2^-103 gives d = 2^-100 exactly for a block whose scale is 8
    and d just below it for scale 7.5; Sg = 2^-120 gives divisors near 2^-114
    and, with subnormal bf16 elements, subnormal fp32 divisors; Sg = 2^124
    gives d above and below 2^125."""
    rng = np.random.default_rng(77)
    out = {}
    sg = 2.0 ** -103
    t = 6.0 * sg
    blocks = [_tie_block(8.0 * sg, 8.0 * t, rng), _tie_block(7.5 * sg, 7.5 * t, rng),
              _tie_block(2.0 ** -100, 6.0 * 2.0 ** -100, rng)]
    out["edge_2m100"] = (to_bf16_bits(np.concatenate(blocks).astype(np.float32)).reshape(1, -1), sg)
    sg = 2.0 ** -120
    blk = _tie_block(44.0 * sg, 2.0 ** -112, rng)
    sub = np.zeros(16)
    sub[0] = 2.0 ** -126
    sub[1] = -(2.0 ** -130)
    sub[2] = 2.0 ** -133
    sub[3] = -(2.0 ** -127)
    out["tiny_global"] = (to_bf16_bits(np.concatenate([blk, sub]).astype(np.float32)).reshape(1, -1), sg)
    sg = 2.0 ** 124
    big = np.full(16, 0.0)
    big[:8] = [3.0e38, -2.0e38, 1.0e38, -5.0e37, 2.5e38, 1.5e38, -3.2e38, 7.0e37]
    mid = _tie_block(0.6875 * sg, 2.0 ** 126, rng)
    out["huge_global"] = (to_bf16_bits(np.concatenate([big, mid]).astype(np.float32)).reshape(1, -1), sg)
    return out


def subnormal_scale_ratio():
    """Dynamic mode, amax 448 (Sg = fl(1/6), t = 1): a block whose maximum
    1.4453125 * 2^-9 rounds to the smallest E4M3 scale 2^-9, so its elements
    reach about 8.7 times the divisor (saturated codes), next to ordinary
    blocks."""
    rng = np.random.default_rng(78)
    amax_blk = rng.standard_normal(16) * 50.0
    amax_blk[5] = 448.0
    b = 1.4453125 * 2.0 ** -9
    odd = rng.uniform(-1.0, 1.0, 16) * b
    odd[0] = b
    odd[1] = -b
    odd[2] = b * 0.93
    return to_bf16_bits(np.concatenate([amax_blk, odd]).astype(np.float32)).reshape(1, -1), None


def all_cases():
    return {
        **extreme_global_scales(),
        "subnormal_scale_ratio": subnormal_scale_ratio(),
        "e2m1_ties": e2m1_ties(),
        "e4m3_ties": e4m3_ties(),
        "scale_edges": scale_edge_cases(),
        "saturation": saturation(),
        "zeros": (np.zeros((2, 32), np.uint16), None),
        "neg_zeros": (np.full((2, 32), 0x8000, np.uint16), None),
    }

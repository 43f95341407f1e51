"""Seeded N(0,1) start for the warm-start factors Q: plain reference.

TEST INFRASTRUCTURE.  Only the tests, the package smoke entry and the
benchmark's CPU-baseline leg import this module; the GPU library never does,
and the two share no code.

The pages start the power iteration from the previous step's Q and leave the
very first Q open; the reading taken here (R10) is i.i.d. standard normal
entries drawn from a counter-based generator keyed by (seed, tensor index), so
every worker that uses the same seed starts from the same Q, whatever the
launch shape or the order the tensors are visited in.

Generator: Philox-4x64 with 10 rounds, as defined in Salmon, Moraes, Dror and
Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11), section 5: each
round multiplies words 0 and 2 by fixed 64-bit constants, and forms the new
words from the high and low halves of the two 128-bit products, the other two
words and the round key; the key is bumped by two Weyl constants between
rounds.  Written with Python integers, so every 128-bit product is exact.

Normal deviates: the Box-Muller transform (Box and Muller, "A note on the
generation of random normal deviates", 1958), computed in float64: two
uniforms u1 in (0, 1] and u2 in [0, 1) give sqrt(-2 ln u1) cos(2 pi u2) and
sqrt(-2 ln u1) sin(2 pi u2).

Layout: Q of a compressed tensor is n x r, stored column by column, and its
element e = c*n + j (row j, column c) is normal number e of the stream keyed
(seed, tensor): Philox block b = e // 4 with counter (b, 0, 0, 0) gives four
words; words 0 and 1 make the normals of e % 4 = 0 and 1, words 2 and 3 those
of e % 4 = 2 and 3.  A column therefore does not depend on the rank.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15  # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B  # sqrt(3) - 1
ROUNDS = 10


def philox4x64(counter: Sequence[int], key: Sequence[int], rounds: int = ROUNDS) -> Tuple[int, int, int, int]:
    """One Philox-4x64 block: four 64-bit words from a 256-bit counter and a
    128-bit key."""
    x0, x1, x2, x3 = (int(c) & MASK64 for c in counter)
    k0, k1 = (int(k) & MASK64 for k in key)
    for rnd in range(rounds):
        if rnd > 0:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        p0 = PHILOX_M0 * x0
        p1 = PHILOX_M1 * x2
        hi0, lo0 = p0 >> 64, p0 & MASK64
        hi1, lo1 = p1 >> 64, p1 & MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return x0, x1, x2, x3


def uniforms(w_a: int, w_b: int) -> Tuple[float, float]:
    """Two 64-bit words -> u1 in (0, 1], u2 in [0, 1), 53 bits each."""
    u1 = 1.0 - (w_a >> 11) * 2.0 ** -53
    u2 = (w_b >> 11) * 2.0 ** -53
    return u1, u2


def box_muller(u1: float, u2: float) -> Tuple[float, float]:
    rad = math.sqrt(-2.0 * math.log(u1))
    ang = 2.0 * math.pi * u2
    return rad * math.cos(ang), rad * math.sin(ang)


def normal_stream(seed: int, tensor: int, count: int) -> np.ndarray:
    """The first `count` normals of the stream keyed (seed, tensor)."""
    out = np.empty(count, np.float64)
    for b in range((count + 3) // 4):
        w = philox4x64((b, 0, 0, 0), (seed, tensor))
        z = box_muller(*uniforms(w[0], w[1])) + box_muller(*uniforms(w[2], w[3]))
        for j in range(4):
            e = 4 * b + j
            if e < count:
                out[e] = z[j]
    return out


def init_q(n: int, rank: int, seed: int, tensor: int) -> np.ndarray:
    """n x rank start Q of tensor `tensor` (reading R10)."""
    flat = normal_stream(seed, tensor, n * rank)
    return flat.reshape(rank, n).T.copy()


def init_q_set(plan, seed: int) -> List[Optional[np.ndarray]]:
    """Start Qs of every compressed tensor of an oracle Plan (None for the
    others)."""
    from .powersgd import KIND_COMPRESSED

    out: List[Optional[np.ndarray]] = []
    for i, kind in enumerate(plan.kinds):
        if kind == KIND_COMPRESSED:
            out.append(init_q(plan.views[i][1], plan.rank, seed, i))
        else:
            out.append(None)
    return out

"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE: part of the CPU oracle.  Only tests/, the smoke check in
__graft_entry__.py and the cpu_baseline leg of bench.py may use this package.

Source of the definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11 -- the Philox-4x32 bijection
with 10 rounds.  One round maps the counter (c0, c1, c2, c3) under key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with M0 = 0xD2511F53, M1 = 0xCD9E8D57, and the key is advanced by the Weyl
constants (0x9E3779B9, 0xBB67AE85) between rounds.

The pages on speculative verification fix only that the verify step draws
independent uniforms (JetSpec++ paper, §3 Preliminaries; App. F.1 Assumption 1(ii)).
How those uniforms are addressed is this library's own convention:

    key     = (lo32(seed), hi32(seed))
    counter = (row i, request b, lo32(offset), hi32(offset))
    u_i     = x0 * 2^-32                          (acceptance uniform, exact in fp64)
    v_i     = (x1 * 2^21 + (x2 >> 11)) * 2^-53    (bonus uniform, 53 bits)

Two implementations live here on purpose: a pure-integer Python one
(`philox4x32_10`) and a vectorised NumPy one (`philox4x32_10_np`).  Tests pin
the first to the published known-answer values and the second to the first.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF
ROUNDS = 10


def philox4x32_10(counter, key):
    """Pure-integer Philox4x32-10 of one 4-word counter under a 2-word key."""
    c0, c1, c2, c3 = (int(x) & _MASK for x in counter)
    k0, k1 = (int(x) & _MASK for x in key)
    for _ in range(ROUNDS):
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & _MASK,
                          (p0 >> 32) ^ c3 ^ k1, p0 & _MASK)
        k0 = (k0 + W0) & _MASK
        k1 = (k1 + W1) & _MASK
    return (c0, c1, c2, c3)


def philox4x32_10_np(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10; every argument broadcasts as uint32."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK for x in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    c0, c1, c2, c3 = (x.copy() for x in (c0, c1, c2, c3))
    k0 = np.uint64(int(k0) & _MASK)
    k1 = np.uint64(int(k1) & _MASK)
    m0, m1 = np.uint64(M0), np.uint64(M1)
    sh, msk = np.uint64(32), np.uint64(_MASK)
    for _ in range(ROUNDS):
        p0 = m0 * c0          # < 2^64: exact in uint64
        p1 = m1 * c2
        n0 = (p1 >> sh) ^ c1 ^ k0
        n1 = p1 & msk
        n2 = (p0 >> sh) ^ c3 ^ k1
        n3 = p0 & msk
        c0, c1, c2, c3 = n0, n1, n2, n3
        k0 = np.uint64((int(k0) + W0) & _MASK)
        k1 = np.uint64((int(k1) + W1) & _MASK)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def uniforms_from_words(x0, x1, x2):
    """(u, v) in [0, 1) from one Philox output, per the convention above."""
    u = float(int(x0)) * 2.0 ** -32
    v = float(int(x1) * 2 ** 21 + (int(x2) >> 11)) * 2.0 ** -53
    return u, v


def block_uniforms(seed: int, offset: int, b: int, i: int):
    """(u_i, v_i) for request b, row i of a verification call keyed by (seed, offset)."""
    seed &= (1 << 64) - 1
    offset &= (1 << 64) - 1
    x0, x1, x2, _ = philox4x32_10((i, b, offset & _MASK, offset >> 32),
                                  (seed & _MASK, seed >> 32))
    return uniforms_from_words(x0, x1, x2)


def block_uniforms_np(seed: int, offset: int, b, i):
    """Vectorised `block_uniforms`: arrays of u and v (float64) for broadcast b, i."""
    seed &= (1 << 64) - 1
    offset &= (1 << 64) - 1
    x0, x1, x2, _ = philox4x32_10_np(i, b, offset & _MASK, offset >> 32,
                                     seed & _MASK, seed >> 32)
    u = x0.astype(np.float64) * 2.0 ** -32
    v = (x1.astype(np.float64) * 2.0 ** 21 + (x2 >> np.uint32(11)).astype(np.float64)) * 2.0 ** -53
    return u, v

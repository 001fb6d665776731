"""Counter-based random numbers for the stochastic-rounding cast.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages do not name a generator ([Drift, "The part I would rather not
write"] only says stochastic rounding carries no bias within one step).  The
cast draws one 32-bit uniform integer per element from Philox4x32-10, the
counter-based generator of Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC11), implemented here from that published
definition:

* state: a 128-bit counter (four 32-bit words c0..c3) and a 64-bit key (k0, k1);
* one round: multiply c0 by 0xD2511F53 and c2 by 0xCD9E8D57 to 64-bit
  products (hi, lo); the new counter is (hi(c2 M1) ^ c1 ^ k0, lo(c2 M1),
  hi(c0 M0) ^ c3 ^ k1, lo(c0 M0));
* between rounds the key is bumped by the Weyl constants (0x9E3779B9,
  0xBB67AE85), modulo 2^32 per word;
* ten rounds; the output is the final counter, four 32-bit words.

Element i of tensor j of a call with 64-bit seed and offset takes word i % 4
of the output for counter (floor(i / 4), j, offset mod 2^32, offset >> 32)
and key (seed mod 2^32, seed >> 32).

Pinned by ``tests/test_oracle_sr.py`` against an independent implementation
(rocRAND's documented Philox4x32-10 interface, run on the host).
"""

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF
ROUNDS = 10


def philox4x32(counter, key, rounds: int = ROUNDS):
    """Tier 0: one block, Python integers."""
    c0, c1, c2, c3 = (int(v) & MASK for v in counter)
    k0, k1 = (int(v) & MASK for v in key)
    for _ in range(rounds):
        p0, p1 = M0 * c0, M1 * c2
        c0, c1, c2, c3 = (p1 >> 32) ^ c1 ^ k0, p1 & MASK, (p0 >> 32) ^ c3 ^ k1, p0 & MASK
        k0, k1 = (k0 + W0) & MASK, (k1 + W1) & MASK
    return c0, c1, c2, c3


def philox4x32_np(c0, c1, c2, c3, k0: int, k1: int, rounds: int = ROUNDS):
    """Tier 1: many blocks at once (arrays of counter words, one key)."""
    c0, c1, c2, c3 = (np.asarray(v, dtype=np.uint64) & np.uint64(MASK) for v in (c0, c1, c2, c3))
    k0, k1 = int(k0) & MASK, int(k1) & MASK
    m = np.uint64(MASK)
    for _ in range(rounds):
        p0 = c0 * np.uint64(M0)          # < 2^64: exact in uint64
        p1 = c2 * np.uint64(M1)
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & m,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & m)
        k0, k1 = (k0 + W0) & MASK, (k1 + W1) & MASK
    return c0, c1, c2, c3


def sr_uniforms(seed: int, offset: int, tensor: int, n: int) -> np.ndarray:
    """The 32-bit uniform integer of each of the n elements of tensor
    `tensor` (its index in the call) under (seed, offset)."""
    nb = (n + 3) // 4
    b = np.arange(nb, dtype=np.uint64)
    z = np.zeros(nb, dtype=np.uint64)
    words = philox4x32_np(b, z + np.uint64(tensor & MASK), z + np.uint64(offset & MASK),
                          z + np.uint64((offset >> 32) & MASK), seed & MASK, (seed >> 32) & MASK)
    return np.stack(words, axis=1).ravel()[:n].astype(np.uint32)


def sr_uniform(seed: int, offset: int, tensor: int, i: int) -> int:
    """Tier 0 form of ``sr_uniforms`` for one element."""
    return philox4x32((i >> 2, tensor, offset & MASK, (offset >> 32) & MASK),
                      (seed & MASK, (seed >> 32) & MASK))[i & 3]


def sr_uniforms_at(seed: int, offset: int, tensor: int, idx: np.ndarray) -> np.ndarray:
    """``sr_uniforms`` at the element indices idx only (sampled checks of
    large tensors)."""
    idx = np.asarray(idx, dtype=np.uint64)
    b = idx >> np.uint64(2)
    z = np.zeros(idx.size, dtype=np.uint64)
    words = philox4x32_np(b & np.uint64(MASK), z + np.uint64(tensor & MASK), z + np.uint64(offset & MASK),
                          z + np.uint64((offset >> 32) & MASK), seed & MASK, (seed >> 32) & MASK)
    w = np.stack(words, axis=1)
    return w[np.arange(idx.size), (idx & np.uint64(3)).astype(np.int64)].astype(np.uint32)

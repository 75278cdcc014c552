"""Counter-based dropout masks that replay exactly in the recompute (oracle).

The pages' mechanism: recomputing a block's forward during the backward would
redraw its dropout masks; Poros avoids that by snapshotting CPU and CUDA RNG
state before each block's forward and restoring it (``torch.random.fork_rng``)
for the recompute ("Poros" research post, the two paragraphs on dropout and RNG
state capture; package README, "How it works").  What is required is that the
recomputed forward sees the identical masks.

Reading taken here: a stateless counter-based generator gives the same
guarantee with no state to snapshot.  The generator is Philox4x32-10 (Salmon,
Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11),
with the round multipliers and Weyl key increments from that paper:

  * key     = (seed mod 2^32, seed >> 32)
  * counter = (e >> 2, (layer << 4) | proj, step, micro), with e = t * K + k the
    row-major element index of the [T, K] LoRA input
  * the element uses output word e & 3
  * keep  <=>  word >= floor(p * 2^32)   (p as fp32, the product in float64)
  * kept elements are scaled by sigma = fp32(1 / fp32(1 - p)) (inverted dropout)

"block" in (seed, block, step) is read as the transformer layer index, so the
masks do not depend on how layers are grouped into streamed windows; proj ids
q 0, k 1, v 2, o 3, gate 4, up 5, down 6 give each projection its own mask.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32 with 10 rounds.

    ctr: four uint32 arrays (broadcastable); key: two uint32 scalars/arrays.
    Returns four uint32 arrays.  Each round: two 32x32->64 products of the
    multipliers with counter words 0 and 2; the new counter is
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key is
    bumped by the Weyl constants between rounds."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK32 for c in ctr)
    k0 = np.asarray(key[0], dtype=np.uint64) & MASK32
    k1 = np.asarray(key[1], dtype=np.uint64) & MASK32
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = np.uint64(M0) * c0
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0), lo1, (hi0 ^ c3 ^ k1), lo0
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def drop_threshold(p: float) -> int:
    """floor(p * 2^32) with p rounded to fp32 first; p must lie in [0, 1)."""
    p32 = float(np.float32(p))
    assert 0.0 <= p32 < 1.0
    return int(np.floor(p32 * 4294967296.0))


def drop_scale(p: float) -> np.float32:
    """sigma = fp32(1 / fp32(1 - p)); exactly 1 at p = 0."""
    one = np.float32(1.0)
    return np.float32(one / np.float32(one - np.float32(p)))


def keep_mask(T: int, K: int, p: float, seed: int, layer: int, proj: int, step: int,
              micro: int) -> np.ndarray:
    """Boolean keep mask [T, K] for one projection's LoRA input."""
    thr = drop_threshold(p)
    if thr == 0:
        return np.ones((T, K), dtype=bool)
    e = np.arange(T * K, dtype=np.uint64)
    ctr = (e >> np.uint64(2), np.uint64(((layer << 4) | proj) & MASK32), np.uint64(step),
           np.uint64(micro))
    key = (seed & MASK32, (seed >> 32) & MASK32)
    words = np.stack(philox4x32_10(ctr, key), axis=0)  # [4, T*K]
    w = words[(e & np.uint64(3)).astype(np.int64), np.arange(T * K)]
    return (w.astype(np.uint64) >= np.uint64(thr)).reshape(T, K)

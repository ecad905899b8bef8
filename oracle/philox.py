"""Philox4x32-10 counter-based generator (oracle).

Test infrastructure only (see ``oracle/__init__``).

Published definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11.  A 128-bit counter
(four 32-bit words) and a 64-bit key (two words) go through 10 rounds; each
round multiplies words 0 and 2 by 0xD2511F53 and 0xCD9E8D57 (full 64-bit
products), and mixes the high halves with the other words and the key; the
key is advanced by the Weyl constants (0x9E3779B9, 0xBB67AE85) between
rounds.

Use in this path (page "Pretraining Large Language Models with NVFP4",
section "2.2" item 4, stochastic rounding of gradients; the page names no
generator -- Philox-4x32 keyed by (seed, element index) is the reading):
* stochastic rounding of element ``idx``: key = (lo32(seed), hi32(seed)),
  counter = (lo32(idx >> 2), hi32(idx >> 2), 0, 0), output word ``idx & 3``;
* the Hadamard sign vector: counter = (0, 0, 1, 0), word 0.
Both equal the ``n``-th output of the stream with subsequence 0 (resp. 1).
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Inputs are uint32-valued arrays / ints;
    returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & MASK for c in (c0, c1, c2, c3))
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for r in range(10):
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        k0 = (k0 + W0) & 0xFFFFFFFF
        k1 = (k1 + W1) & 0xFFFFFFFF
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def stream_words(seed: int, idx, subsequence: int = 0) -> np.ndarray:
    """Word ``idx & 3`` of block ``idx >> 2`` of the keyed stream."""
    idx = np.asarray(idx, dtype=np.uint64)
    blk = idx >> np.uint64(2)
    w = philox4x32_10(blk & MASK, blk >> np.uint64(32),
                      subsequence & 0xFFFFFFFF, subsequence >> 32,
                      seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    sel = (idx & np.uint64(3)).astype(np.int64)
    return np.choose(sel, w).astype(np.uint32)

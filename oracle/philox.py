"""Philox4x32-10 and the stochastic-rounding bit mapping (oracle; test infrastructure only).

Philox4x32-10 is written from its published definition (Salmon et al.,
"Parallel random numbers: as easy as 1, 2, 3", SC'11): a 4x32-bit counter and
a 2x32-bit key; each of the 10 rounds multiplies counter words 0 and 2 by the
constants 0xD2511F53 and 0xCD9E8D57 into 64-bit products, and the new counter
is (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)).  The key
is bumped by the Weyl constants (0x9E3779B9, 0xBB67AE85) between rounds.

The pages ask for stochastic rounding ("MXFP4", AI Wiki, §Training with
MXFP4; "Training an MoE LLM in MXFP4", summary) but fix neither the generator
nor how bits are assigned to elements.  The reading taken (one written rule so
that two independent implementations can agree bit for bit):

  * each element takes 16 random bits;
  * element p (flat index in the quantized output's logical [rows_out, K]
    order) uses Philox call q = p >> 3 with counter
    (q mod 2^32, q >> 32, offset mod 2^32, offset >> 32) and key
    (seed mod 2^32, seed >> 32);
  * its bits are the 16-bit half (p & 1) (0 = low half) of output word
    ((p >> 1) & 3).

The bits therefore do not depend on launch geometry, and quantizing X along
dim 0 gives the same bits as quantizing X^T along its last dim.

An 8-bit variant ("sr8", an option beside the 16-bit default) spends one
Philox call on 16 elements: element p uses call q = p >> 4 (the same counter
and key layout) and takes byte (p & 3) of output word ((p >> 2) & 3).
"""

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Vectorised Philox4x32-10.  Counter words c0..c3 are uint32 arrays (or
    scalars); key words k0, k1 are Python ints.  Returns four uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for rnd in range(10):
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
        if rnd != 9:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
    return tuple(w.astype(np.uint32) for w in (c0, c1, c2, c3))


def sr_bits16(p, seed, offset):
    """The 16 random bits of output element(s) at flat index p (uint64 array)."""
    p = np.asarray(p, dtype=np.uint64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    q = p >> np.uint64(3)
    w = philox4x32_10(q & MASK32, q >> np.uint64(32),
                      np.uint64(offset & 0xFFFFFFFF), np.uint64(offset >> 32),
                      seed & 0xFFFFFFFF, seed >> 32)
    words = np.stack(w, axis=0).astype(np.uint64)          # [4, ...]
    sel = ((p >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(words, sel[None, ...], axis=0)[0]
    half = (p & np.uint64(1)) * np.uint64(16)
    return ((word >> half) & np.uint64(0xFFFF)).astype(np.uint32)


def sr_bits8(p, seed, offset):
    """The 8 random bits of output element(s) at flat index p (uint64 array)
    under the 8-bit mapping: byte (p & 3) of word ((p >> 2) & 3) of Philox
    call p >> 4."""
    p = np.asarray(p, dtype=np.uint64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    offset = int(offset) & 0xFFFFFFFFFFFFFFFF
    q = p >> np.uint64(4)
    w = philox4x32_10(q & MASK32, q >> np.uint64(32),
                      np.uint64(offset & 0xFFFFFFFF), np.uint64(offset >> 32),
                      seed & 0xFFFFFFFF, seed >> 32)
    words = np.stack(w, axis=0).astype(np.uint64)
    sel = ((p >> np.uint64(2)) & np.uint64(3)).astype(np.int64)
    word = np.take_along_axis(words, sel[None, ...], axis=0)[0]
    shift = (p & np.uint64(3)) * np.uint64(8)
    return ((word >> shift) & np.uint64(0xFF)).astype(np.uint32)

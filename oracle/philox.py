"""Philox4x64-10 and the uniform draws of one ISD step (oracle side).

Test infrastructure: a plain Python implementation written from the
published definition of Philox (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11, section 3: the Philox S-box built from
one wide multiply per word pair, a Weyl-sequence key schedule, ten rounds).
It shares nothing with the HIP generator; the pin is numpy's own Philox
bit generator (a library routine) and the all-zero known-answer block.

The pages only say that acceptance uniforms come from a seeded stream
(I-DLM, fr.news.hada.io, "Documentation et ressources > Inference & ISD"
states the min(1, p/q) test; the variant and counter layout are not given).
Reading adopted here:
  key     = (seed, 0)
  counter = (slot, sequence, step, 0)
  u       = ((word0 >> 41) + 0.5) * 2**-23
so u = (2k+1) * 2**-24 with a 23-bit k: never 0 or 1 and exact in fp32 and
fp64, which lets the kernel and the oracle compare the very same u.
Slots of one step: 1..N-1 test the drafts, N draws the final (bonus or
residual) token, N+k draws proposal k (k = 1..N-1). Slot 0 is unused.
"""

import numpy as np

MASK64 = (1 << 64) - 1
# Multipliers and key increments of Philox4x64 (SC'11, table 2).
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15  # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B  # sqrt(3) - 1


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for one 256-bit counter block."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in counter)
    k0, k1 = (int(x) & MASK64 for x in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        prod0 = PHILOX_M0 * c0
        prod1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = (
            (prod1 >> 64) ^ c1 ^ k0,
            prod1 & MASK64,
            (prod0 >> 64) ^ c3 ^ k1,
            prod0 & MASK64,
        )
    return c0, c1, c2, c3


def uniform_from_word(word):
    """Map the top 23 bits of a 64-bit word to (k + 0.5) / 2**23."""
    return ((int(word) >> 41) + 0.5) / float(1 << 23)


def step_uniforms(seed, step, C, N):
    """Uniforms u[b, slot] for one step: float64 array of shape [C, 2N]."""
    u = np.empty((C, 2 * N), dtype=np.float64)
    for b in range(C):
        for slot in range(2 * N):
            w = philox4x64_10((slot, b, step, 0), (seed, 0))[0]
            u[b, slot] = uniform_from_word(w)
    return u

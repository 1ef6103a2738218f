"""Tokens per forward (TPF) of the strided decoding loop (oracle side).

Test infrastructure. The pages give, for the memory-bound regime, speedup
approximately TPF = (2 + p + ... + p^(N-2)) / (2 - p^(N-1)) with acceptance
rate p and stride N, and quote TPF about 2.9 with efficiency TPF^2 /
query_size = 1.22 at N = 4, p = 0.9 (I-DLM, fr.news.hada.io, "Throughput" and
"Speedup Factor Explorer"; efficiency defined on papoo.work).

The chain below is the two-state model of the accept loop that this closed
form describes: a FULL step runs N-1 draft tests, each passing with
probability p independently; if all pass it emits N tokens and stays FULL,
if the first failure is test j it emits j tokens and goes FRESH; a FRESH
step emits one token and goes FULL. Its long-run ratio of tokens to forwards
is the closed form exactly (renewal reward theorem).
"""

import numpy as np


def tpf_closed_form(N, p):
    """(2 + p + ... + p^(N-2)) / (2 - p^(N-1)); the sum is empty for N = 2."""
    num = 2.0 + sum(p ** k for k in range(1, N - 1))
    return num / (2.0 - p ** (N - 1))


def efficiency(tpf, query_size):
    """TPF^2 / query size."""
    return tpf * tpf / query_size


def tpf_chain(N, p, steps, rng):
    """Simulate the FULL/FRESH chain with Bernoulli(p) tests; returns
    (tokens per forward, accepted-length histogram over FULL steps)."""
    nd = N - 1
    full = False
    tokens = 0
    hist = np.zeros(N, np.int64)
    for _ in range(steps):
        if not full:
            tokens += 1
            full = True
            continue
        tests = rng.random(nd) < p
        a = nd if tests.all() else int(np.argmin(tests))
        hist[a] += 1
        tokens += a + 1
        full = a == nd
    return tokens / steps, hist

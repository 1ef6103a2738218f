"""Seeded synthetic inputs of the ISD step, shared by the tests, the benchmark
and the oracle checks.

This module draws random numbers and lays them out; it holds none of the
method's arithmetic (no softmax, acceptance test, attention or projection).
Everything is a deterministic function of the seed, so the kernel side and
the oracle side of a test receive identical bytes.

The pages describe no throughput workload (their benchmarks need trained
weights), so the inputs stand in with the shapes the pages' model family
implies: grouped-query attention of 8B/32B-class models (Qwen3-8B/32B bases,
I-DLM, fr.news.hada.io, "Documentation et ressources > Model Zoo"), a
151,936-entry vocabulary, stride N = 4 at concurrency 64 ("Aperçu").
"""

import hashlib

import numpy as np
import torch

PAGE_SIZE = 16

# Draft-noise standard deviations that give a mean acceptance of about 0.5,
# 0.7 and 0.9 for logits ~ N(0, 3^2) over 151,936 entries rounded to bf16.
# Written by oracle/calibrate_noise.py (which calls only the oracle); the
# values it measured are stored in tests/golden/noise_sigma.json.
SIGMA_Q_V151936 = {0.5: 1.3539, 0.7: 0.7637, 0.9: 0.2477}


def seed_of(*parts):
    """A 63-bit seed mixed from integers and strings."""
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*parts))
    return g


def normal(shape, std, dtype, device, *seed_parts):
    """N(0, std^2) samples drawn in float32 and rounded to dtype."""
    g = _gen(device, *seed_parts)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def contexts(seed, C, ctx):
    """Per-sequence cached lengths: an int, a list, or ("uniform", lo, hi)."""
    if isinstance(ctx, tuple) and ctx and ctx[0] == "uniform":
        rng = np.random.default_rng(seed_of(seed, "ctx"))
        return rng.integers(ctx[1], ctx[2] + 1, size=C).astype(np.int32)
    arr = np.broadcast_to(np.asarray(ctx, dtype=np.int32), (C,))
    return arr.copy()


def block_table(seed, capacity, spare_pages=0, page_size=PAGE_SIZE):
    """Pages for capacity[b] positions per sequence, placed by a seeded
    shuffle of a free list. Unused table entries hold -1."""
    need = (np.asarray(capacity, np.int64) + page_size - 1) // page_size
    total = int(need.sum()) + int(spare_pages)
    rng = np.random.default_rng(seed_of(seed, "pages"))
    perm = rng.permutation(total).astype(np.int32)
    max_pages = int(need.max()) if len(need) else 0
    table = np.full((len(need), max(max_pages, 1)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, total


class AttentionCase:
    """One attention workload: queries of the stride block and the logical
    K/V rows of every sequence (positions 0 .. ctx_b + rows - 1)."""

    def __init__(self, seed, C, rows, Hq, Hkv, D, ctx, dtype=torch.bfloat16,
                 spare_pages=0, headroom=0, device="cpu"):
        self.C, self.rows, self.Hq, self.Hkv, self.D = C, rows, Hq, Hkv, D
        self.dtype = dtype
        self.ctx = contexts(seed, C, ctx)
        self.lengths = self.ctx + rows
        self.table, self.num_pages = block_table(
            seed, self.lengths + headroom, spare_pages)
        Lmax = int(self.lengths.max())
        self.q = normal((C, rows, Hq, D), 1.0, dtype, device, seed, "q")
        self.k_rows = normal((C, Lmax, Hkv, D), 1.0, dtype, device, seed, "k")
        self.v_rows = normal((C, Lmax, Hkv, D), 1.0, dtype, device, seed, "v")


class TeacherLogits:
    """Synthetic stand-in for the LM head over a stride block.

    A fixed table T[b, i] ~ N(0, sigma_l^2) plays the AR model's logits for
    the token at position ctx0_b + 1 + i of sequence b. A block row r of a
    sequence with ctx cached tokens predicts position ctx + r + 1 (logit
    shift); a clean row (r <= n_draft) returns T at that position, a MASK row
    (r > n_draft) returns T plus fresh N(0, sigma_q^2) noise drawn per step.
    So a draft proposed from a MASK row is later verified against the noise-
    free row of the same position, and the noise sets the acceptance rate.
    """

    def __init__(self, seed, C, V, n_positions, sigma_l, sigma_q,
                 dtype=torch.bfloat16, device="cpu"):
        self.seed, self.C, self.V = seed, C, V
        self.sigma_q = sigma_q
        self.dtype, self.device = dtype, device
        self.table = normal((C, n_positions, V), sigma_l, dtype, device,
                            seed, "teacher")

    def block(self, step, ctx, ctx0, n_draft, rows):
        """Logits [C, rows, V] for one step; ctx, ctx0, n_draft are int
        tensors on the generator's device (no host synchronisation)."""
        C = self.C
        idx = (ctx - ctx0).long()[:, None] + torch.arange(rows, device=self.device)[None, :]
        if self.device == "cpu" and int(idx.max()) >= self.table.shape[1]:
            raise ValueError("teacher table too short for this position")
        out = torch.gather(self.table, 1, idx[:, :, None].expand(C, rows, self.V))
        noise = normal((C, rows, self.V), self.sigma_q, torch.float32,
                       self.device, self.seed, "mask-noise", int(step))
        is_mask = (torch.arange(rows, device=self.device)[None, :]
                   > n_draft.long()[:, None])
        noisy = (out.float() + noise).to(self.dtype)
        return torch.where(is_mask[:, :, None], noisy, out)


def lora_case(seed, M, K, Nout, r, dtype=torch.bfloat16, device="cpu",
              w_std=0.02, ab_std=0.01):
    """Projection inputs: x ~ N(0,1), W ~ N(0, w_std^2), A, B ~ N(0, ab_std^2)."""
    x = normal((M, K), 1.0, dtype, device, seed, "x")
    W = normal((Nout, K), w_std, dtype, device, seed, "W")
    A = normal((r, K), ab_std, dtype, device, seed, "A")
    B = normal((Nout, r), ab_std, dtype, device, seed, "B")
    return x, W, A, B


def stride_mask(M, N):
    """MASK rows of a batch of 2N-row stride blocks: rows N..2N-1 of each."""
    return (np.arange(M) % (2 * N)) >= N


def step_outputs(seed, C, N, V, bad_frac=0.0):
    """Synthetic per-sequence state and step outputs (int32 numpy arrays),
    shaped like what one accept step leaves behind: n_draft in {0, N-1},
    drafts, emit with n_emit valid entries (-1 after), ctx after the commit.
    A fraction bad_frac of the sequences gets an invalid n_draft or
    n_emit."""
    rng = np.random.default_rng(seed_of(seed, "step-outputs"))
    n_draft = np.where(rng.random(C) < 0.7, N - 1, 0).astype(np.int32)
    drafts = rng.integers(0, V, (C, N - 1)).astype(np.int32)
    drafts[n_draft == 0] = -1
    n_emit = rng.integers(1, N + 1, C).astype(np.int32)
    emit = rng.integers(0, V, (C, N)).astype(np.int32)
    emit[np.arange(N)[None, :] >= n_emit[:, None]] = -1
    ctx = rng.integers(0, 32768, C).astype(np.int32)
    bad = rng.random(C) < bad_frac
    kind = rng.integers(0, 3, C)
    n_draft[bad & (kind == 0)] = 1 if N > 2 else -1   # neither FULL nor FRESH
    n_emit[bad & (kind == 1)] = 0                     # step not taken
    n_emit[bad & (kind == 2)] = N + 1
    return n_draft, drafts, emit, n_emit, ctx

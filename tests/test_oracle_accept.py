"""Pins of the oracle's accept step (CPU only).

Each test checks the oracle against something other than itself: the
closed-form tokens per forward printed on the pages, the distribution the
p/q rule must preserve, brute force, and special cases with known answers.
"""

import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import accept, chain, philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def logits_of(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, dtype=np.float64))


def full_state(C, N, drafts, q_row=1):
    return (np.full(C, N - 1), np.asarray(drafts).reshape(C, N - 1), np.full(C, q_row))


# ---------------------------------------------------------------- inverse CDF

def brute_inv_cdf(w, u):
    total = sum(w)
    run = 0.0
    for v, x in enumerate(w):
        run += x
        if run > u * total:
            return v
    raise AssertionError


@pytest.mark.parametrize("seed", range(20))
def test_inv_cdf_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    w = rng.random(13) * (rng.random(13) < 0.7)
    if w.sum() == 0:
        w[3] = 1.0
    for u in rng.random(50):
        assert accept.inv_cdf(w, u)[0] == brute_inv_cdf(w, u)


def test_inv_cdf_special_cases():
    assert accept.inv_cdf([0, 0, 1.0, 0], 0.999)[0] == 2
    assert accept.inv_cdf([0, 0, 0.3, 0.7], 1e-9)[0] == 2
    # strict '>' with ascending ids: a threshold exactly on a cumulative sum
    # goes to the next id
    assert accept.inv_cdf([0.5, 0.5], 0.5)[0] == 1
    v, margin = accept.inv_cdf([0.25, 0.25, 0.5], 0.3)
    assert v == 1 and margin == pytest.approx(0.05)


# ------------------------------------------------------------ the p/q test

def one_full_step(P_rows, Q_rows, drafts, u, N):
    """FULL step for C sequences with verify rows P_rows [n+1.., V] used as
    rows 0..N-1, proposal rows after them, and the pending drafts' q rows in
    the previous block at rows 1..N-1."""
    C = u.shape[0]
    V = P_rows.shape[-1]
    R = 2 * N
    cur = np.zeros((C, R, V))
    cur[:, :N] = logits_of(P_rows)
    cur[:, N:] = 0.0
    prev = np.zeros((C, R, V))
    prev[:, 1:N] = logits_of(Q_rows)
    n, d, qr = full_state(C, N, drafts)
    return accept.accept_step(cur, prev, n, d, qr, u, N)


def test_p_equal_q_accepts_every_draft():
    rng = np.random.default_rng(0)
    N, V, C = 4, 50, 40
    rows = rng.dirichlet(np.ones(V), size=N)
    P = np.broadcast_to(rows, (C, N, V))
    Q = np.broadcast_to(rows[:N - 1], (C, N - 1, V))
    drafts = rng.integers(0, V, (C, N - 1))
    u = philox.step_uniforms(5, 0, C, N)
    out = one_full_step(P, Q, drafts, u, N)
    assert (out["accepted"] == N - 1).all()
    assert (out["n_emit"] == N).all() and (out["kv_commit"] == N).all()
    assert (out["n_draft_next"] == N - 1).all() and (out["q_row_next"] == N).all()
    assert (out["emit"][:, :N - 1] == drafts).all()


def test_accept_rate_is_sum_of_min():
    """E[accept] = sum_x min(P, Q) when x ~ Q (the identity behind the
    AR-preservation claim)."""
    rng = np.random.default_rng(1)
    V, N, C = 6, 2, 20000
    P = rng.dirichlet(np.ones(V))
    Q = rng.dirichlet(np.ones(V))
    x = rng.choice(V, size=C, p=Q)
    u = rng.random((C, 2 * N))
    out = one_full_step(np.broadcast_to(P, (C, N, V)), np.broadcast_to(Q, (C, 1, V)), x[:, None], u, N)
    rate = out["accepted"].mean()
    expect = np.minimum(P, Q).sum()
    assert abs(rate - expect) < 4 * np.sqrt(expect * (1 - expect) / C)


def test_one_hot_q_accepts_with_probability_p_of_x():
    rng = np.random.default_rng(2)
    V, N, C = 5, 2, 20000
    P = rng.dirichlet(np.ones(V))
    Q = np.zeros(V)
    Q[3] = 1.0
    u = rng.random((C, 2 * N))
    out = one_full_step(np.broadcast_to(P, (C, N, V)), np.broadcast_to(Q, (C, 1, V)),
                        np.full((C, 1), 3), u, N)
    rate = out["accepted"].mean()
    assert abs(rate - P[3]) < 4 * np.sqrt(P[3] * (1 - P[3]) / C)
    # after a rejection the residual max(0, P - Q) puts no mass on id 3
    rej = out["accepted"] == 0
    assert rej.any() and (out["emit"][rej, 0] != 3).all()


def test_first_emitted_token_is_distributed_as_p_chi2():
    """The rejection sampler as a whole (test + residual) emits its first
    token from P_0, whatever Q is."""
    rng = np.random.default_rng(3)
    V, N, C = 8, 2, 40000
    P = rng.dirichlet(np.ones(V) * 0.7)
    Q = rng.dirichlet(np.ones(V) * 0.7)
    x = rng.choice(V, size=C, p=Q)
    u = rng.random((C, 2 * N))
    out = one_full_step(np.broadcast_to(P, (C, N, V)), np.broadcast_to(Q, (C, 1, V)), x[:, None], u, N)
    counts = np.bincount(out["emit"][:, 0], minlength=V)
    keep = P * C > 5
    chi2, pval = stats.chisquare(counts[keep], P[keep] / P[keep].sum() * counts[keep].sum())
    assert pval > 1e-4, (chi2, pval)


def test_first_emitted_token_exact_enumeration():
    """V = 3, N = 2: enumerate the draft over Q and both uniforms over a
    midpoint grid; the emitted token's law must be P_0 to grid accuracy."""
    P = np.array([0.5, 0.3, 0.2])
    Q = np.array([0.2, 0.2, 0.6])
    N, G = 2, 48
    grid = (np.arange(G) + 0.5) / G
    prob = np.zeros(3)
    for x in range(3):
        uu = np.zeros((G * G, 2 * N))
        uu[:, 1] = np.repeat(grid, G)
        uu[:, N] = np.tile(grid, G)
        C = G * G
        out = one_full_step(np.broadcast_to(P, (C, N, 3)), np.broadcast_to(Q, (C, 1, 3)),
                            np.full((C, 1), x), uu, N)
        prob += Q[x] * np.bincount(out["emit"][:, 0], minlength=3) / C
    assert np.allclose(prob, P, atol=2.0 / G)


def test_second_emitted_token_given_first_accepted_is_p1():
    rng = np.random.default_rng(4)
    V, N, C = 6, 3, 30000
    P = rng.dirichlet(np.ones(V), size=N)
    Q = rng.dirichlet(np.ones(V), size=N - 1)
    drafts = np.stack([rng.choice(V, size=C, p=Q[j]) for j in range(N - 1)], 1)
    u = rng.random((C, 2 * N))
    out = one_full_step(np.broadcast_to(P, (C, N, V)), np.broadcast_to(Q, (C, N - 1, V)), drafts, u, N)
    sel = out["accepted"] >= 1
    counts = np.bincount(out["emit"][sel, 1], minlength=V)
    chi2, pval = stats.chisquare(counts, P[1] * counts.sum())
    assert pval > 1e-4, (chi2, pval)
    # the bonus after all drafts pass comes from the last verify row
    sel = out["accepted"] == N - 1
    counts = np.bincount(out["emit"][sel, N - 1], minlength=V)
    chi2, pval = stats.chisquare(counts, P[N - 1] * counts.sum())
    assert pval > 1e-4, (chi2, pval)


def test_rejection_returns_fresh_state_and_bonus_follows_full():
    P = np.array([[0.0, 1.0], [0.5, 0.5]])
    Q = np.array([[1.0, 0.0]])
    u = np.full((1, 4), 0.5)
    out = one_full_step(P[None], Q[None], np.array([[0]]), u, 2)
    # P(0) = 0 so the draft 0 is rejected; residual is one-hot on id 1
    assert out["accepted"][0] == 0 and out["emit"][0, 0] == 1
    assert out["n_draft_next"][0] == 0 and out["kv_commit"][0] == 1
    assert out["resid_mass"][0] == pytest.approx(1.0)


def test_fresh_step_emits_bonus_and_proposes():
    N, V = 4, 7
    rng = np.random.default_rng(6)
    cur = rng.normal(size=(1, 2 * N, V))
    u = philox.step_uniforms(3, 1, 1, N)
    out = accept.accept_step(cur, None, np.zeros(1, int), np.full((1, N - 1), -1), np.zeros(1, int), u, N)
    assert out["accepted"][0] == 0 and out["n_emit"][0] == 1 and out["kv_commit"][0] == 1
    assert out["emit"][0, 0] == accept.inv_cdf(accept.softmax(cur[0, 0]), u[0, N])[0]
    for k in range(1, N):
        assert out["drafts_next"][0, k - 1] == accept.inv_cdf(accept.softmax(cur[0, k]), u[0, N + k])[0]
    assert out["q_row_next"][0] == 1 and out["n_draft_next"][0] == N - 1


# ------------------------------------------------ tokens per forward (pages)

def test_closed_form_matches_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "pages_tpf.json")))
    row = g["printed"][0]
    tpf = chain.tpf_closed_form(row["N"], row["p"])
    assert abs(tpf - row["tpf_approx"]) < 0.05
    assert chain.efficiency(tpf, 2 * row["N"] - 1) == pytest.approx(row["efficiency"], abs=0.005)
    # limits: every draft accepted -> N per forward; none -> 1 per forward
    for N in range(2, 9):
        assert chain.tpf_closed_form(N, 1.0) == pytest.approx(N)
        assert chain.tpf_closed_form(N, 0.0) == pytest.approx(1.0)


@pytest.mark.parametrize("N,p", [(4, 0.9), (4, 0.5), (2, 0.9), (8, 0.7), (3, 0.5), (6, 0.9), (6, 0.5)])
def test_bernoulli_chain_reproduces_closed_form(N, p):
    rng = np.random.default_rng(N * 100 + int(p * 10))
    steps = 200000
    tpf, _ = chain.tpf_chain(N, p, steps, rng)
    # per-forward token counts are bounded by N; a crude 5-sigma band
    assert abs(tpf - chain.tpf_closed_form(N, p)) < 5 * N / np.sqrt(steps) + 0.01


@pytest.mark.parametrize("N,p", [(4, 0.9), (3, 0.7), (2, 0.5), (6, 0.9), (8, 0.7)])
def test_oracle_accept_loop_reproduces_closed_form(N, p):
    """Run the oracle's own accept step as a decoding loop over C sequences:
    clean rows are a fixed P, MASK rows a fixed Q with sum min(P, Q) = p, so
    each draft passes independently with probability p."""
    d = 1.0 - p
    P = np.array([0.5, 0.5])
    Q = np.array([0.5 + d, 0.5 - d])
    lp, lq = logits_of(P), logits_of(Q)
    C, steps, R = 48, 160, 2 * N
    n = np.zeros(C, int)
    drafts = np.full((C, N - 1), -1)
    q_row = np.zeros(C, int)
    prev = None
    tokens = 0
    for step in range(steps):
        cur = np.empty((C, R, 2))
        r = np.arange(R)[None, :, None]
        cur[:] = np.where(r <= n[:, None, None], lp, lq)
        u = philox.step_uniforms(99, step, C, N)
        out = accept.accept_step(cur, prev, n, drafts, q_row, u, N)
        tokens += out["n_emit"].sum()
        n, drafts, q_row, prev = out["n_draft_next"], out["drafts_next"], out["q_row_next"], cur
    tpf = tokens / (C * steps)
    assert abs(tpf - chain.tpf_closed_form(N, p)) < 0.08, tpf


def test_flagged_marks_near_boundary_draws():
    out = {"accepted": np.array([0, 0]),
           "accept_margin": np.array([[2e-6, np.inf], [0.3, np.inf]]),
           "final_margin": np.array([0.1, 0.1]),
           "propose_margin": np.array([[np.inf, np.inf], [0.2, 5e-7]])}
    assert accept.flagged(out).tolist() == [True, True]
    out["propose_margin"][1, 1] = 0.2
    assert accept.flagged(out).tolist() == [True, False]


# ------------------------------------------------ argmax proposals (reading)

def argmax_step(P_rows, Q_rows, u, N):
    """FULL step with argmax proposals: the drafts are argmax of the q rows."""
    drafts = np.argmax(Q_rows, axis=-1)
    C = u.shape[0]
    V = P_rows.shape[-1]
    R = 2 * N
    cur = np.zeros((C, R, V))
    cur[:, :N] = logits_of(P_rows)
    prev = np.zeros((C, R, V))
    prev[:, 1:N] = logits_of(Q_rows)
    n, d, qr = full_state(C, N, drafts)
    return accept.accept_step(cur, prev, n, d, qr, u, N, proposal="argmax"), drafts


def test_argmax_first_emitted_token_exact_enumeration():
    """A point-mass proposal still leaves the first emitted token distributed
    as P_0: enumerate both uniforms over a midpoint grid (V = 4, N = 2)."""
    P = np.array([0.1, 0.4, 0.3, 0.2])
    Q = np.array([0.1, 0.2, 0.6, 0.1])  # argmax 2
    N, G = 2, 64
    grid = (np.arange(G) + 0.5) / G
    C = G * G
    uu = np.zeros((C, 2 * N))
    uu[:, 1] = np.repeat(grid, G)
    uu[:, N] = np.tile(grid, G)
    out, drafts = argmax_step(np.broadcast_to(P, (C, N, 4)), np.broadcast_to(Q, (C, 1, 4)), uu, N)
    assert (drafts == 2).all()
    prob = np.bincount(out["emit"][:, 0], minlength=4) / C
    assert np.allclose(prob, P, atol=2.0 / G)
    # acceptance is P(x) exactly (to the grid), and a rejection never emits x
    assert abs(out["accepted"].mean() - P[2]) <= 1.0 / G
    assert (out["emit"][out["accepted"] == 0, 0] != 2).all()
    assert np.allclose(out["q_x"][:, 0], 1.0)


def test_argmax_proposals_and_residual_mass():
    rng = np.random.default_rng(11)
    V, N, C = 7, 3, 4000
    P = rng.dirichlet(np.ones(V), size=N)
    Q = rng.dirichlet(np.ones(V), size=N - 1)
    u = rng.random((C, 2 * N))
    out, drafts = argmax_step(np.broadcast_to(P, (C, N, V)), np.broadcast_to(Q, (C, N - 1, V)), u, N)
    # chi-square of the first emitted token against P_0
    counts = np.bincount(out["emit"][:, 0], minlength=V)
    chi2, pval = stats.chisquare(counts, P[0] * C)
    assert pval > 1e-4, (chi2, pval)
    # the residual after rejecting x_1 is P_0 without x_1: its mass is 1 - P_0(x_1)
    rej = out["accepted"] == 0
    x1 = int(np.argmax(Q[0]))
    assert np.allclose(out["resid_mass"][rej], 1.0 - P[0][x1])
    # new drafts, when all pass, are the argmax of the proposal rows
    full = out["accepted"] == N - 1
    assert full.any()
    assert np.isinf(out["propose_margin"][full]).all() and np.allclose(out["q_x_next"][full], 1.0)


def test_argmax_loop_reproduces_closed_form():
    """Decoding loop with argmax proposals where every draft passes with
    probability p = P(argmax Q): tokens per forward follows the pages'
    closed form at that p."""
    N, p = 4, 0.7
    P = np.array([p, 1.0 - p])
    Q = np.array([0.8, 0.2])  # argmax 0, accepted with probability P[0] = p
    lp, lq = logits_of(P), logits_of(Q)
    C, steps, R = 48, 160, 2 * N
    n = np.zeros(C, int)
    drafts = np.full((C, N - 1), -1)
    q_row = np.zeros(C, int)
    prev = None
    tokens = 0
    for step in range(steps):
        cur = np.empty((C, R, 2))
        r = np.arange(R)[None, :, None]
        cur[:] = np.where(r <= n[:, None, None], lp, lq)
        u = philox.step_uniforms(77, step, C, N)
        out = accept.accept_step(cur, prev, n, drafts, q_row, u, N, proposal="argmax")
        tokens += out["n_emit"].sum()
        n, drafts, q_row, prev = out["n_draft_next"], out["drafts_next"], out["q_row_next"], cur
    tpf = tokens / (C * steps)
    assert abs(tpf - chain.tpf_closed_form(N, p)) < 0.08, tpf


# ------------------------------------------------------------ block assembly

MASK = 151669  # any id outside the synthetic vocabularies below


def test_block_assemble_layout_examples():
    """The stride block layout (the FULL/FRESH reading): written out by hand
    for N = 4 and N = 2, not computed."""
    N = 4
    tokens, pos, is_mask = accept.block_assemble(
        n_draft=[3, 0, 3], drafts=[[11, 12, 13], [-1, -1, -1], [7, 8, 9]],
        emit=[[21, 22, 23, 40], [50, -1, -1, -1], [60, -1, -1, -1]], n_emit=[4, 1, 1],
        ctx=[100, 7, 0], N=N, mask_id=MASK)
    M = MASK
    assert tokens.tolist() == [[40, 11, 12, 13, M, M, M, M],   # FULL: [t, d1..d3, MASK x 4]
                               [50, M, M, M, M, M, M, M],      # FRESH: [t, MASK x 7]
                               [60, 7, 8, 9, M, M, M, M]]
    assert pos.tolist() == [list(range(100, 108)), list(range(7, 15)), list(range(0, 8))]
    assert is_mask.tolist() == [[False] * 4 + [True] * 4, [False] + [True] * 7, [False] * 4 + [True] * 4]
    tokens, _, is_mask = accept.block_assemble([1, 0], [[5], [-1]], [[3, 4], [6, -1]], [2, 1], [9, 9], 2, MASK)
    assert tokens.tolist() == [[4, 5, M, M], [6, M, M, M]]
    # a step not taken (n_emit 0) or a state that is neither FULL nor FRESH
    tokens, _, is_mask = accept.block_assemble([3, 1], [[1, 2, 3], [1, 2, 3]], [[-1] * 4, [5, -1, -1, -1]],
                                               [0, 1], [4, 4], 4, MASK)
    assert (tokens == -1).all() and not is_mask.any()


@pytest.mark.parametrize("N", [2, 4])
def test_block_assemble_feeds_the_cache_every_emitted_token_once(N):
    """An oracle decoding loop in which each step's block comes from
    block_assemble: the tokens the KV cache commits (rows 0..a of each block)
    are exactly the emitted stream, in order, one token late, and row 0 of
    every block sits at the position of that token in the stream. The
    drafts of each block are the ones the next accept step verifies."""
    V, C, steps, R = 6, 16, 40, 2 * N
    rng = np.random.default_rng(5)
    ctx0 = rng.integers(10, 50, C)
    # clean rows: a fixed P per position; MASK rows: a nearby Q
    P = rng.dirichlet(np.ones(V), size=(C, 200))
    Q = 0.6 * P + 0.4 * rng.dirichlet(np.ones(V), size=(C, 200))
    ctx = ctx0.copy()
    n = np.zeros(C, int)
    drafts = np.full((C, N - 1), -1)
    q_row = np.zeros(C, int)
    # step 0's block is the prompt's last token followed by MASK rows
    first = rng.integers(0, V, C)
    tokens = np.full((C, R), MASK)
    tokens[:, 0] = first
    is_mask = np.broadcast_to(np.arange(R)[None, :] > 0, (C, R))
    prev = None
    emitted = [[int(first[b])] for b in range(C)]  # the stream: prompt's last token, then emits
    committed = [[] for _ in range(C)]
    for step in range(steps):
        for b in range(C):  # the block carries the drafts this step verifies
            assert tokens[b, 1:1 + n[b]].tolist() == drafts[b, :n[b]].tolist()
        pos = ctx[:, None] + np.arange(R)[None, :]
        cur = np.empty((C, R, V))
        for b in range(C):
            for i in range(R):
                src = Q if is_mask[b, i] else P
                cur[b, i] = logits_of(src[b, pos[b, i] - ctx0[b] + 1])
        u = philox.step_uniforms(17, step, C, N)
        out = accept.accept_step(cur, prev, n, drafts, q_row, u, N)
        for b in range(C):
            committed[b] += tokens[b, : out["kv_commit"][b]].tolist()
            emitted[b] += out["emit"][b, : out["n_emit"][b]].tolist()
        ctx = ctx + out["kv_commit"]
        n, drafts, q_row, prev = out["n_draft_next"], out["drafts_next"], out["q_row_next"], cur
        tokens, positions, is_mask = accept.block_assemble(n, drafts, out["emit"], out["n_emit"], ctx, N, MASK)
        for b in range(C):
            # row 0 is the newest emitted token, at its index in the stream
            assert tokens[b, 0] == emitted[b][-1]
            assert positions[b, 0] == ctx0[b] + len(emitted[b]) - 1
        assert (is_mask.sum(1) == np.where(n == N - 1, N, 2 * N - 1)).all()
    for b in range(C):
        assert committed[b] == emitted[b][:-1]


# ------------------------------------------------- chunked softmax statistics

def test_chunk_stats_brute_force_and_row_normaliser():
    """Per-run (max, sum exp(l - max)) by plain loops, the last run short;
    merged over the runs they give the row's own softmax normaliser."""
    import math
    rng = np.random.default_rng(11)
    for V, chunk in ((37, 8), (64, 16), (100, 100), (5, 8)):
        row = rng.normal(0.0, 3.0, V) + 40.0  # large logits: the shift by the max matters
        got = accept.chunk_stats(row, chunk)
        assert got.shape == (-(-V // chunk), 2)
        for c in range(got.shape[0]):
            part = [float(x) for x in row[c * chunk:(c + 1) * chunk]]
            m = max(part)
            s = math.fsum(math.exp(x - m) for x in part)
            assert got[c, 0] == m
            assert abs(got[c, 1] - s) <= 1e-12 * s
        M = float(np.max(row))
        merged = math.fsum(math.exp(m - M) * s for m, s in got)
        assert abs(merged - math.fsum(math.exp(float(x) - M) for x in row)) <= 1e-12 * merged


def test_chunk_stats_special_cases():
    """Equal entries give (value, count); -inf entries add nothing."""
    got = accept.chunk_stats(np.array([2.0, 2.0, 2.0, -np.inf, 1.0, -np.inf]), 3)
    assert got[0, 0] == 2.0 and got[0, 1] == 3.0
    assert got[1, 0] == 1.0 and got[1, 1] == 1.0

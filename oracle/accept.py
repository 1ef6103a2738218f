"""The accept side of one ISD step: verify, resample, propose (oracle side).

Test infrastructure, plain numpy in float64; it shares no code with the HIP
path. What the pages fix, and where:

* One causal forward both verifies the drafts of the previous step and
  proposes new tokens (I-DLM, fr.news.hada.io, "Aperçu" and "Méthodologie
  d'I-DLM > Introspective Strided Decoding (ISD)"; abstract on fugumt.com).
* Proposals q come from MASK positions, verification p from clean positions,
  and a draft x is kept with probability min(1, p(x)/q(x)), which keeps the
  AR distribution (same page, "Documentation et ressources > Inference &
  ISD").
* Causal attention plus a logit shift: the output of row i is the
  distribution of the token at position i+1 (same page, "Méthodologie
  d'I-DLM > Entraînement à la cohérence introspective").
* The tokens-per-forward closed form of "Speedup Factor Explorer" is what the
  step structure below reproduces (see oracle.chain).

Readings where the pages are silent (each one is listed with its reason in
the design notes):
* Block of R = 2N rows. FULL state (n = N-1 pending drafts):
  [b, d_1..d_{N-1}, MASK x N]; FRESH state (n = 0): [r, MASK x (2N-1)].
  Row j-1 verifies draft j; row n gives the bonus; rows n+1..n+N-1 propose.
* Rejection sampling in its standard form: on the first rejection, draw from
  normalize(max(0, P_a - Q_{a+1})); if that mass is zero, draw from P_a.
  After all n drafts pass, draw a bonus token from P_n and propose N-1 new
  drafts; after a rejection the MASK proposals are void (they were made
  after a rejected token) and the next step is FRESH.
* accept iff u * Q(x) < P(x) (u in (0,1), never 0 or 1).
* inverse CDF over ascending token ids with a strict '>' test.
* KV commit = a + 1 rows (row 0 and the accepted drafts), emitted = a + 1.
* temperature 1, full vocabulary.
"""

import numpy as np


def softmax(row):
    """Stable softmax of one logits row (float64)."""
    row = np.asarray(row, dtype=np.float64)
    m = np.max(row)
    e = np.exp(row - m)
    return e / e.sum()


def row_stats(row):
    """(max, sum of exp(l - max)) of one logits row, float64."""
    row = np.asarray(row, dtype=np.float64)
    m = np.max(row)
    return m, float(np.exp(row - m).sum())


def chunk_stats(row, chunk):
    """(max, sum of exp(l - max)) of each run of `chunk` consecutive entries
    of one logits row (the last run may be shorter), float64, shape [n, 2].

    The softmax normaliser of the row is a sum over its entries, so it splits
    over any partition of the vocabulary: with M the row maximum,
    sum_v exp(l_v - M) = sum_c exp(m_c - M) * s_c for the runs' (m_c, s_c).
    Computing the runs where the logits are produced (the LM-head GEMM) is
    the same quantity as row_stats, re-associated.
    """
    row = np.asarray(row, dtype=np.float64)
    out = []
    for c0 in range(0, row.shape[0], chunk):
        out.append(row_stats(row[c0:c0 + chunk]))
    return np.array(out, dtype=np.float64)


def inv_cdf(w, u):
    """Smallest index v with sum_{v' <= v} w[v'] > u * sum(w).

    Returns (index, margin): margin is the distance, in the units of w, from
    the threshold to the nearer of the two cumulative sums that bracket it.
    """
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    t = u * c[-1]
    v = int(np.searchsorted(c, t, side="right"))
    if v >= len(w):  # only reachable through rounding when u is near 1
        v = int(np.flatnonzero(w > 0)[-1])
    lo = c[v - 1] if v > 0 else 0.0
    margin = min(t - lo, c[v] - t)
    return v, float(margin)


def accept_step(logits, prev_logits, n_draft, drafts, q_row, u, N, proposal="sample"):
    """One accept step for a batch of C sequences.

    proposal "sample" (the default): drafts are drawn from the MASK rows'
    softmax q and verified with min(1, p/q). proposal "argmax": the pages'
    serving stack proposes argmax q instead (I-DLM, fr.news.hada.io,
    "Documentation et ressources > Serving (SGLang)": argmax proposal); q is
    then a point mass at the draft, so the same rule reads accept iff
    u < p(x), and the residual max(0, p - q) is p with the draft removed.
    (The pages do not spell out that rule; it is the standard rejection step
    with a point-mass proposal.) Ties of the argmax go to the smallest id.

    logits      float64 [C, R, V]   this step's block logits (R >= 2N-1 used)
    prev_logits float64 [C, R', V]  the previous step's block (q rows of the
                                    pending drafts), or None if no drafts
    n_draft     int [C]             pending drafts per sequence (0..N-1)
    drafts      int [C, N-1]        pending draft ids
    q_row       int [C]             row of prev_logits that proposed draft 1
                                    (draft j came from row q_row + j - 1)
    u           float64 [C, 2N]     uniforms by slot (see oracle.philox)

    Returns a dict of per-sequence outputs and diagnostics; see the keys.
    """
    logits = np.asarray(logits, dtype=np.float64)
    C, R, V = logits.shape
    nd = N - 1
    out = {
        "accepted": np.zeros(C, np.int64),
        "n_emit": np.zeros(C, np.int64),
        "emit": np.full((C, N), -1, np.int64),
        "kv_commit": np.zeros(C, np.int64),
        "n_draft_next": np.zeros(C, np.int64),
        "drafts_next": np.full((C, nd), -1, np.int64),
        "q_row_next": np.zeros(C, np.int64),
        # probabilities the pass criteria name
        "p_x": np.full((C, nd), np.nan),       # P_{j-1}(x_j)
        "q_x": np.full((C, nd), np.nan),       # Q_j(x_j)
        "q_x_next": np.full((C, nd), np.nan),  # Q(x') of the new drafts
        "resid_mass": np.full(C, np.nan),      # sum max(0, P_a - Q_{a+1})
        # per-row softmax statistics of the rows this step reads
        "row_m": np.full((C, R), np.nan),
        "row_s": np.full((C, R), np.nan),
        # margins of every decision this step takes (see module notes)
        "accept_margin": np.full((C, nd), np.inf),
        "final_margin": np.full(C, np.inf),
        "propose_margin": np.full((C, nd), np.inf),
    }
    for b in range(C):
        n = int(n_draft[b])
        assert 0 <= n <= nd
        last_row = n + nd  # rows 0..n verify/bonus, n+1..n+N-1 propose
        assert last_row < R
        for r in range(last_row + 1):
            out["row_m"][b, r], out["row_s"][b, r] = row_stats(logits[b, r])
        P = [softmax(logits[b, j]) for j in range(n + 1)]

        def q_dist(j):
            row = prev_logits[b, int(q_row[b]) + j - 1]
            if proposal == "argmax":
                q = np.zeros(V)
                q[int(np.argmax(row))] = 1.0
                return q
            return softmax(row)

        a = 0
        for j in range(1, n + 1):
            x = int(drafts[b, j - 1])
            px = P[j - 1][x]
            qx = q_dist(j)[x]
            out["p_x"][b, j - 1] = px
            out["q_x"][b, j - 1] = qx
            if qx > 0:
                out["accept_margin"][b, j - 1] = abs(u[b, j] - px / qx)
            if u[b, j] * qx < px:
                a += 1
            else:
                break

        if a < n:
            w = np.maximum(0.0, P[a] - q_dist(a + 1))
            out["resid_mass"][b] = w.sum()
            if w.sum() == 0.0:
                w = P[a]
            t, margin = inv_cdf(w, u[b, N])
            out["final_margin"][b] = margin
            out["n_draft_next"][b] = 0
            out["q_row_next"][b] = 0
        else:
            t, margin = inv_cdf(P[n], u[b, N])
            out["final_margin"][b] = margin
            for k in range(1, N):
                if proposal == "argmax":
                    # exact comparisons of the same values on both sides:
                    # no boundary to be near
                    xk, qx, mk = int(np.argmax(logits[b, n + k])), 1.0, np.inf
                else:
                    Qk = softmax(logits[b, n + k])
                    xk, mk = inv_cdf(Qk, u[b, N + k])
                    qx = Qk[xk]
                out["drafts_next"][b, k - 1] = xk
                out["q_x_next"][b, k - 1] = qx
                out["propose_margin"][b, k - 1] = mk
            out["n_draft_next"][b] = nd
            out["q_row_next"][b] = n + 1

        out["accepted"][b] = a
        out["n_emit"][b] = a + 1
        out["kv_commit"][b] = a + 1
        out["emit"][b, :a] = drafts[b, :a]
        out["emit"][b, a] = t
    return out


def flagged(out, tol=1e-5):
    """Per-sequence flag: some decision this step took lay within tol of its
    boundary (accept margin |u - P/Q|, or a CDF margin in probability
    units), so a kernel computing in another precision may decide otherwise.
    """
    C = out["accepted"].shape[0]
    flag = np.zeros(C, bool)
    for b in range(C):
        tested = out["accept_margin"][b]
        if np.any(tested[np.isfinite(tested)] < tol):
            flag[b] = True
        if out["final_margin"][b] < tol:
            flag[b] = True
        pm = out["propose_margin"][b]
        if np.any(pm[np.isfinite(pm)] < tol):
            flag[b] = True
    return flag


def block_assemble(n_draft, drafts, emit, n_emit, ctx, N, mask_id):
    """The next step's stride block of every sequence (I-DLM,
    fr.news.hada.io, "Méthodologie d'I-DLM > Introspective Strided Decoding
    (ISD)": each forward carries the clean tokens still to be verified and
    MASK positions for the next proposals).

    Reading (the block layout above): row 0 is the last token the step
    emitted (the bonus or the resampled token, not yet in the KV cache),
    rows 1..n are the n pending drafts, the other rows of the 2N are MASK:
    FULL (n = N-1) gives [t, d_1..d_{N-1}, MASK x N], FRESH (n = 0) gives
    [t, MASK x (2N-1)]. Row i sits at position ctx + i, with ctx taken after
    the commit. A sequence whose step was not taken (n_emit < 1) or whose
    state is not FULL or FRESH gets -1 tokens and no MASK rows.

    n_draft [C], drafts [C, N-1], emit [C, N], n_emit [C], ctx [C] (ints)
    Returns tokens [C, 2N], positions [C, 2N], is_mask [C, 2N] (bool).
    """
    C = len(n_draft)
    R = 2 * N
    tokens = np.full((C, R), -1, np.int64)
    positions = np.zeros((C, R), np.int64)
    is_mask = np.zeros((C, R), bool)
    for b in range(C):
        positions[b] = int(ctx[b]) + np.arange(R)
        n, ne = int(n_draft[b]), int(n_emit[b])
        if n not in (0, N - 1) or not 1 <= ne <= N:
            continue
        tokens[b, 0] = emit[b][ne - 1]
        for i in range(1, R):
            if i <= n:
                tokens[b, i] = drafts[b][i - 1]
            else:
                tokens[b, i] = mask_id
                is_mask[b, i] = True
    return tokens, positions, is_mask

"""GPU parity of isd_lm_head, and isd_accept fed with its statistics.

Pass criteria: each logit (stored in bf16, the type the accept step reads)
within one bf16 rounding of the fp64 oracle product, i.e. 2^-8 relative
(bf16 keeps 8 significant bits; the fp32 accumulation adds far less);
chunk maxima equal to the maxima of the stored logits, chunk sums within
1e-5 relative of the oracle's sums over the stored logits; rows computed
with other rows or alone give the same bits; isd_accept given these
statistics takes the same decisions as with its own statistics pass, except
on a draw the oracle finds within 1e-5 of its boundary.
"""

import numpy as np
import pytest
import torch

import draft_verify_decoding_amd as dvd
import workload
from oracle import accept as ref
from oracle import lora as lin
from oracle import philox

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHUNK = 8192


def case(seed, M, K, V, sigma_w):
    print(f"lm head case M={M} K={K} V={V}", flush=True)
    h = workload.normal((M, K), 1.0, torch.bfloat16, "cpu", seed, "lm-h")
    W = workload.normal((V, K), sigma_w, torch.bfloat16, "cpu", seed, "lm-W")
    return h, W


def check_rows(logits, stats, want, rows):
    """logits [n, V] bf16 and stats [n, nch, 2] of the given rows against the
    fp64 product want [n, V]."""
    got = logits.float().double().numpy()
    # one bf16 rounding (half a unit in the last of 8 significant bits) of
    # an fp32 sum whose own error is orders of magnitude smaller
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-5 * np.abs(want).max())
    st = stats.double().numpy()
    for i, r in enumerate(rows):
        o = ref.chunk_stats(got[i], CHUNK)
        assert np.array_equal(st[i, :, 0], o[:, 0]), r
        rel = np.abs(st[i, :, 1] - o[:, 1]) / o[:, 1]
        assert rel.max() < 1e-5, (r, rel.max())


@pytest.mark.parametrize("V", [20000, 8192, 100])
def test_lm_head_matches_oracle_ragged(V):
    """40 rows (not a multiple of any tile), ragged last tile and chunk."""
    M, K = 40, 256
    h, W = case(1, M, K, V, 0.1)
    logits, stats = dvd.isd_lm_head(h.to(DEV), W.to(DEV))
    torch.cuda.synchronize()
    assert stats.shape == (M, -(-V // CHUNK), 2)
    want = lin.linear(h.double().numpy(), W.double().numpy())
    check_rows(logits.cpu(), stats.cpu(), want, range(M))


def test_lm_head_rows_do_not_depend_on_the_batch():
    """Rows 24..31 computed alone (another tile shape and grid) keep their
    logits and statistics bit for bit."""
    M, K, V = 512, 512, 30000
    h, W = case(2, M, K, V, 0.1)
    hd, Wd = h.to(DEV), W.to(DEV)
    lg, st = dvd.isd_lm_head(hd, Wd)
    lg1, st1 = dvd.isd_lm_head(hd[24:32].contiguous(), Wd)
    torch.cuda.synchronize()
    assert torch.equal(lg[24:32].view(torch.int16), lg1.view(torch.int16))
    assert torch.equal(st[24:32].view(torch.int32), st1.view(torch.int32))


def test_lm_head_at_the_8b_shape_sampled_rows():
    """512 rows (C=64, 2N=8), hidden 4096, vocabulary 151,936, written with a
    padded row stride: sampled rows against the oracle, padding untouched."""
    M, K, V, ld = 512, 4096, 151936, 151936 + 64
    h, W = case(3, M, K, V, 0.03)
    hd, Wd = h.to(DEV), W.to(DEV)
    buf = torch.full((M, ld), float("nan"), dtype=torch.bfloat16, device=DEV)
    lg, st = dvd.isd_lm_head(hd, Wd, logits=buf[:, :V])
    torch.cuda.synchronize()
    assert torch.isnan(buf[:, V:].float()).all()
    rows = np.array([0, 1, 7, 100, 255, 256, 510, 511])
    want = lin.linear(h[rows].double().numpy(), W.double().numpy())
    check_rows(lg.cpu()[rows], st.cpu()[rows], want, rows)


def test_accept_with_lm_head_statistics():
    """Three steps of isd_accept on LM-head logits (C=16, N=4, V=20000),
    run twice in lockstep: with the LM head's chunk statistics and with the
    accept's own statistics pass. Same decisions, emitted ids and next
    state, except where the oracle finds a draw within 1e-5 of its boundary;
    and the statistics path equals the oracle, fed the same state, on the
    accepted length, emitted ids, commit, next drafts and their q(x)."""
    C, N, V, K = 16, 4, 20000, 256
    R = 2 * N
    seed = 5
    Wd = workload.normal((V, K), 0.15, torch.bfloat16, "cpu", seed, "acc-W").to(DEV)
    sa_in, sa_out = dvd.SeqState(C, N), dvd.SeqState(C, N)
    sb_in, sb_out = dvd.SeqState(C, N), dvd.SeqState(C, N)
    prev = None
    active = np.ones(C, bool)
    excused = 0
    checked = 0
    for step in range(3):
        print(f"lm head accept step {step}", flush=True)
        # verify rows of this step lean on last step's MASK rows so that some drafts pass
        h = workload.normal((C * R, K), 1.0, torch.float32, "cpu", seed, "acc-h", step)
        if prev is not None:
            h[:, :] = 0.7 * prev_h + 0.3 * h
        prev_h = h.clone()
        lg, st = dvd.isd_lm_head(h.to(torch.bfloat16).to(DEV), Wd)
        lg = lg.view(C, R, V)
        st = st.view(C, R, -1, 2)
        n_before = sb_in.n_draft.cpu().numpy().copy()
        drafts_before = sb_in.drafts.cpu().numpy().copy()
        qrow_before = sb_in.q_row.cpu().numpy().copy()
        oa = dvd.isd_accept(lg, prev, sa_in, sa_out, N, seed, step, diag=True, chunk_stats=st)
        ob = dvd.isd_accept(lg, prev, sb_in, sb_out, N, seed, step, diag=True)
        torch.cuda.synchronize()
        o = ref.accept_step(lg.float().double().cpu().numpy(), None if prev is None else prev.float().double().cpu().numpy(),
                            n_before.astype(np.int64), drafts_before.astype(np.int64), qrow_before.astype(np.int64),
                            philox.step_uniforms(seed, step, C, N), N)
        flags = ref.flagged(o, 1e-5)
        for b in np.flatnonzero(active):
            same = all(np.array_equal(getattr(oa, k).cpu().numpy()[b], getattr(ob, k).cpu().numpy()[b])
                       for k in ("accepted", "n_emit", "emit", "kv_commit"))
            same = same and all(np.array_equal(getattr(sa_out, k).cpu().numpy()[b], getattr(sb_out, k).cpu().numpy()[b])
                                for k in ("n_draft", "drafts", "q_row"))
            if not same:
                assert flags[b], (step, b)
                active[b] = False
                excused += 1
                continue
            # the LM-head-statistics path agrees with the oracle on the same
            # inputs: accepted length, emitted ids, commit, the next state
            # and the q(x) of new drafts (1e-5), unless a draw was flagged
            if not flags[b]:
                assert int(oa.accepted.cpu()[b]) == int(o["accepted"][b]), (step, b)
                assert int(oa.kv_commit.cpu()[b]) == int(o["kv_commit"][b]), (step, b)
                assert np.array_equal(oa.emit.cpu().numpy()[b], o["emit"][b]), (step, b)
                assert int(sa_out.n_draft.cpu()[b]) == int(o["n_draft_next"][b]), (step, b)
                assert int(sa_out.q_row.cpu()[b]) == int(o["q_row_next"][b]), (step, b)
                if o["n_draft_next"][b] == N - 1:
                    assert np.array_equal(sa_out.drafts.cpu().numpy()[b], o["drafts_next"][b]), (step, b)
                    assert np.all(np.abs(sa_out.q_x.cpu().numpy()[b] - o["q_x_next"][b]) <= 1e-5), (step, b)
                checked += 1
            pa, pb = oa.p_x.cpu().numpy()[b], ob.p_x.cpu().numpy()[b]
            ok = np.isfinite(pb)
            assert np.all(np.abs(pa[ok] - pb[ok]) <= 1e-5)
            both = ok & np.isfinite(o["p_x"][b])
            assert np.all(np.abs(pa[both] - o["p_x"][b][both]) <= 1e-5)
        sa_in, sa_out = sa_out, sa_in
        sb_in, sb_out = sb_out, sb_in
        prev = lg
    assert active.sum() >= C - 2, excused
    # rows of 20,000 flat-ish entries put many draws within 1e-5 of a CDF
    # boundary (flagged, so not compared); at least C sequence-steps are
    assert checked >= C, checked

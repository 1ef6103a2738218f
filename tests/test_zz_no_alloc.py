"""isd_accept_noalloc (the accept step for callers that cannot allocate
device memory) against isd_accept on the same inputs: two calls in a row,
the second with fewer sequences and a smaller vocabulary, both compared bit
for bit on every output and the next state. Called through the C ABI."""

import numpy as np
import pytest
import torch

import draft_verify_decoding_amd as dvd
import workload

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_pair(C, N, V, seed, steps):
    """`steps` accept steps along one trajectory, each computed twice from
    the same inputs: through isd_accept with its own workspace and through
    isd_accept_noalloc. Every output must match bit for bit."""
    print(f"no-alloc accept C={C} N={N} V={V} steps={steps}", flush=True)
    R = 2 * N
    teacher = workload.TeacherLogits(seed, C, V, steps * N + R + 1, 3.0, 0.3, torch.bfloat16, DEV)
    ctx0 = torch.zeros(C, dtype=torch.int64, device=DEV)
    ctx = ctx0.clone()
    s_in, s_a, s_b = dvd.SeqState(C, N, DEV), dvd.SeqState(C, N, DEV), dvd.SeqState(C, N, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    prev = None
    for t in range(steps):
        lg = teacher.block(t, ctx, ctx0, s_in.n_draft.long(), R).contiguous()
        oa = dvd.isd_accept(lg, prev, s_in, s_a, N, seed, t, diag=True, dev_err=err)
        ob = dvd.AcceptOutputs(C, N, R, DEV, diag=True)
        dvd.isd_accept(lg, prev, s_in, s_b, N, seed, t, out=ob, diag=True, dev_err=err, noalloc=True)
        torch.cuda.synchronize()
        assert err.item() == 0
        for k in ("accepted", "n_emit", "emit", "kv_commit", "p_x", "resid_mass", "row_m", "row_s"):
            x, y = getattr(oa, k), getattr(ob, k)
            if x.is_floating_point():
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), (t, k)
        for k in ("n_draft", "drafts", "q_x", "q_m", "q_s", "q_row"):
            x, y = getattr(s_a, k), getattr(s_b, k)
            if x.is_floating_point():
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), (t, k)
        ctx += oa.kv_commit.long()
        prev = lg
        s_in.copy_(s_a)
    return int((ctx - ctx0).sum())


def test_noalloc_accept_equals_accept_on_two_calls_in_a_row():
    # first call: the 8B bench shape; second: fewer sequences, smaller vocabulary
    emitted = run_pair(64, 4, 151936, 11, 3)
    assert emitted > 64 * 3
    emitted = run_pair(5, 3, 3000, 12, 3)
    assert emitted >= 5 * 3


def test_noalloc_rejects_a_call_beyond_its_scratch():
    lib = dvd.lib()
    cap = int(lib.isd_accept_noalloc_max_workspace())
    assert dvd.isd_accept_workspace_size(64, 4, 151936, 8) <= cap
    C = 65535  # stats of 65,535 x 16 rows x 64 chunks do not fit
    assert dvd.isd_accept_workspace_size(C, 8, 524288, 16) > cap
    lg = torch.zeros((1, 16, 8), dtype=torch.bfloat16, device=DEV)
    s_in, s_out = dvd.SeqState(1, 8, DEV), dvd.SeqState(1, 8, DEV)
    out = dvd.AcceptOutputs(1, 8, 16, DEV, diag=False)
    args = dvd.IsdAcceptArgs()
    args.C, args.N, args.V, args.rows, args.dtype = C, 8, 524288, 16, dvd.ISD_BF16
    args.logits, args.ld = lg.data_ptr(), 524288
    args.in_, args.out = s_in.c_struct(), s_out.c_struct()
    args.accepted, args.n_emit = out.accepted.data_ptr(), out.n_emit.data_ptr()
    args.emit, args.kv_commit = out.emit.data_ptr(), out.kv_commit.data_ptr()
    rc = lib.isd_accept_noalloc(args, None)
    assert rc == -3  # ISD_E_WORKSPACE, nothing launched

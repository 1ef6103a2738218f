"""GPU edge cases at the limits of each call: the most sequences one
attention call takes, the largest vocabulary and the most sequences of the
accept step, partial KV writes, and the smallest projection. Each output is
compared with the oracle to the same bars as the main parity tests."""

import numpy as np
import pytest
import torch

import draft_verify_decoding_amd as dvd
import workload
from oracle import attention as ref_att
from oracle import lora as ref_lora

from test_gpu_accept import run_trajectory
from test_gpu_attention import fill_cache, slab_errors, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_attention_most_sequences_per_call():
    """8192 sequences (the per-call limit) with contexts 0..40: one launch
    plans all of them; a sample of sequences is checked in full."""
    C = 8192
    print(f"attention C={C}", flush=True)
    case = workload.AttentionCase(61, C=C, rows=8, Hq=4, Hkv=1, D=64, ctx=("uniform", 0, 40))
    kv, err = fill_cache(case)
    out = dvd.isd_attention(kv, case.q.to(DEV), torch.from_numpy(case.ctx).to(DEV),
                            max_len=int(case.lengths.max()), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    got = out.cpu().double().numpy()
    seqs = np.array([0, 1, 777, 4095, 4096, 8190, 8191])
    kp = np.zeros((case.num_pages, 16, case.Hkv, case.D))
    vp = np.zeros_like(kp)
    ref_att.kv_write(kp, vp, case.table[seqs], np.zeros(len(seqs), int), to64(case.k_rows[seqs]),
                     to64(case.v_rows[seqs]), case.lengths[seqs])
    want = ref_att.block_attention(to64(case.q[seqs]), kp, vp, case.table[seqs], case.ctx[seqs])
    assert slab_errors(got[seqs], want).max() < 2e-3


def test_kv_write_partial_rows_and_offsets():
    """nrows below rows (including 0) and non-zero start positions: only the
    named rows land, at the named positions; every other slot keeps its
    value."""
    C, rows, Hkv, D = 3, 8, 2, 128
    case = workload.AttentionCase(62, C=C, rows=rows, Hq=4, Hkv=Hkv, D=D, ctx=[20, 33, 7], headroom=8)
    kv = dvd.KVCache(case.num_pages, Hkv, D, torch.bfloat16, torch.from_numpy(case.table), DEV)
    kv.k_pages.fill_(7.0)
    kv.v_pages.fill_(-3.0)
    k = workload.normal((C, rows, Hkv, D), 1.0, torch.bfloat16, "cpu", 62, "pk")
    v = workload.normal((C, rows, Hkv, D), 1.0, torch.bfloat16, "cpu", 62, "pv")
    pos0 = np.array([20, 33, 7], np.int32)
    nrows = np.array([8, 3, 0], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dvd.isd_kv_write(kv, k.to(DEV), v.to(DEV), torch.from_numpy(pos0).to(DEV), torch.from_numpy(nrows).to(DEV),
                     dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    P = case.num_pages
    kd = to64(kv.k_pages).reshape(P, Hkv, D // 8, 16, 8)
    vd = to64(kv.v_pages).reshape(P, Hkv, 2, D, 8)
    written = np.zeros((P, 16), bool)
    for b in range(C):
        for r in range(nrows[b]):
            t = pos0[b] + r
            p, s = case.table[b, t // 16], t % 16
            written[p, s] = True
            assert np.array_equal(kd[p, :, :, s, :].reshape(Hkv, D), to64(k[b, r]))
            assert np.array_equal(vd[p, :, s // 8, :, s % 8], to64(v[b, r]))
    for p in range(P):
        for s in range(16):
            if not written[p, s]:
                assert (kd[p, :, :, s, :] == 7.0).all() and (vd[p, :, s // 8, :, s % 8] == -3.0).all()


def test_kv_write_negative_start_writes_the_valid_rows():
    """A block that starts at position -2 flags ISD_DEV_STATE for its first
    two rows and writes the others at positions 0, 1, 2; nothing else moves."""
    Hkv, D, rows = 2, 64, 5
    case = workload.AttentionCase(66, C=1, rows=rows, Hq=2, Hkv=Hkv, D=D, ctx=[0], headroom=16)
    kv = dvd.KVCache(case.num_pages, Hkv, D, torch.bfloat16, torch.from_numpy(case.table), DEV)
    kv.k_pages.fill_(7.0)
    kv.v_pages.fill_(-3.0)
    k = workload.normal((1, rows, Hkv, D), 1.0, torch.bfloat16, "cpu", 66, "nk")
    v = workload.normal((1, rows, Hkv, D), 1.0, torch.bfloat16, "cpu", 66, "nv")
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dvd.isd_kv_write(kv, k.to(DEV), v.to(DEV), torch.tensor([-2], dtype=torch.int32, device=DEV), dev_err=err)
    torch.cuda.synchronize()
    assert err.item() & dvd.DEV_STATE
    P = case.num_pages
    kd = to64(kv.k_pages).reshape(P, Hkv, D // 8, 16, 8)
    vd = to64(kv.v_pages).reshape(P, Hkv, 2, D, 8)
    p0 = case.table[0, 0]
    for t in range(16):
        if t < 3:
            assert np.array_equal(kd[p0, :, :, t, :].reshape(Hkv, D), to64(k[0, t + 2]))
            assert np.array_equal(vd[p0, :, t // 8, :, t % 8], to64(v[0, t + 2]))
        else:
            assert (kd[p0, :, :, t, :] == 7.0).all() and (vd[p0, :, t // 8, :, t % 8] == -3.0).all()


def test_accept_largest_vocabulary():
    """V = 524,288 (the largest the chunk-statistics cache takes), bf16."""
    t, _ = run_trajectory(3, seed=63, C=2, N=2, V=524288, sigma_l=3.0, sigma_q=0.3,
                          dtype=torch.bfloat16, ctx0=10)
    assert t.compared >= 4


def test_accept_many_sequences_small_vocabulary():
    """4096 sequences in one call, vocabulary 64, stride 3."""
    t, _ = run_trajectory(3, seed=64, C=4096, N=3, V=64, sigma_l=2.0, sigma_q=0.5,
                          dtype=torch.float32, ctx0=0)
    assert t.compared >= 3 * 4096 - 20


@pytest.mark.parametrize("M,K,Nout,r", [(1, 64, 16, 128), (7, 64, 33, 16)])
def test_smallest_projections(M, K, Nout, r):
    x, W, A, B = workload.lora_case(65, M, K, Nout, r)
    mask = np.arange(M) % 2 == 1
    xd, Wd, Ad, Bd = (t.to(DEV).contiguous() for t in (x, W, A, B))
    md = torch.from_numpy(mask.astype(np.uint8)).to(DEV)
    base = dvd.isd_linear(xd, Wd)
    y = dvd.isd_linear_gated(xd, Wd, Ad, Bd, md, scale=0.7)
    torch.cuda.synchronize()
    want = ref_lora.gated_lora(x.double().numpy(), W.double().numpy(), A.double().numpy(), B.double().numpy(),
                               mask, 0.7)
    got = y.cpu().double().numpy()
    assert np.abs(got - want).max() / np.abs(want).max() < 2e-3
    m = torch.from_numpy(mask).to(DEV)
    assert torch.equal(y[~m].view(torch.int32), base[~m].view(torch.int32))


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_kv_write_keeps_every_other_slot(dtype, D):
    """Pools filled with random values; blocks that start inside a half page,
    cross a half page, cross a page and start on a page boundary, with 8, 3,
    1 and 8 rows, are written: the written slots hold the rows (documented
    layout: K [page][head][D/KP][16 slots][KP], V [page][head][2 halves][D]
    [8 slots]) and every other element of both pools keeps its bits."""
    Hkv, rows = 2, 8
    pos0 = np.array([5, 13, 16, 30], dtype=np.int32)
    nrows = np.array([8, 3, 1, 8], dtype=np.int32)
    case = workload.AttentionCase(67, C=4, rows=rows, Hq=2, Hkv=Hkv, D=D, ctx=pos0.tolist(), dtype=dtype)
    kv = dvd.KVCache(case.num_pages, Hkv, D, dtype, torch.from_numpy(case.table), DEV)
    kv.k_pages.copy_(workload.normal(tuple(kv.k_pages.shape), 1.0, dtype, "cpu", 67, "kpool").to(DEV))
    kv.v_pages.copy_(workload.normal(tuple(kv.v_pages.shape), 1.0, dtype, "cpu", 67, "vpool").to(DEV))
    k = workload.normal((4, rows, Hkv, D), 1.0, dtype, "cpu", 67, "k")
    v = workload.normal((4, rows, Hkv, D), 1.0, dtype, "cpu", 67, "v")
    P, KP = case.num_pages, 16 // (2 if dtype == torch.bfloat16 else 4)
    want_k = kv.k_pages.cpu().clone().reshape(P, Hkv, D // KP, 16, KP)
    want_v = kv.v_pages.cpu().clone().reshape(P, Hkv, 2, D, 8)
    for b in range(4):
        for r in range(int(nrows[b])):
            pos = int(pos0[b]) + r
            page, slot = case.table[b, pos // 16], pos % 16
            want_k[page, :, :, slot, :] = k[b, r].reshape(Hkv, D // KP, KP)
            want_v[page, :, slot // 8, :, slot % 8] = v[b, r]
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    dvd.isd_kv_write(kv, k.to(DEV), v.to(DEV), torch.from_numpy(pos0).to(DEV), torch.from_numpy(nrows).to(DEV),
                     dev_err=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert torch.equal(kv.k_pages.cpu().reshape(want_k.shape), want_k)
    assert torch.equal(kv.v_pages.cpu().reshape(want_v.shape), want_v)
